/* Hardware-rate probes for gfx950 (MI355X), libtilemix_probes.so.
 *
 * Timing-only kernels behind the kernels' cost model: vector-ALU issue
 * rates, the matrix pipe beside the vector ALU, direct HBM->LDS copies, LDS
 * read rates and the HBM read patterns of the decode step.  They compute
 * nothing of the attention path and no entry point of libtilemix.so calls
 * them.  Each launches one kernel on `stream` (a hipStream_t, NULL for the
 * default stream) and returns at once: 0 on success, -1 for an argument out
 * of range (nothing launched), -2 when the launch failed.  `out` is a device
 * buffer the kernels never write in practice (they store only a value their
 * work cannot produce); it must hold blocks * 512 elements (blocks * 256 for
 * tilemix_probe_valu and tilemix_probe_read's 1,024 groups), except for
 * tilemix_probe_clock, which writes its four counters.  The caller
 * times the launches (events on the same stream). */
#ifndef TILEMIX_PROBES_H
#define TILEMIX_PROBES_H

#ifdef __cplusplus
extern "C" {
#endif

/* Rows and heads of each operand of tilemix_probe_read: k and v are device
 * buffers of exactly ROWS * HEADS * 128 bytes (32 MiB). */
#define TILEMIX_PROBE_READ_ROWS 32768
#define TILEMIX_PROBE_READ_HEADS 8

/* 16 independent chains per thread of op 0 (fp32 FMA) or 1 (v_exp_f32),
 * `iters` steps each, `blocks` groups of 256 threads (blocks / 256 waves per
 * SIMD when the groups spread evenly over the 256 CUs). */
int tilemix_probe_valu(int op, int blocks, int iters, float* out, void* stream);

/* One 512-thread group per CU: waves 0-3 run four 32x32x16 f16 MFMA chains,
 * waves 4-7 eight fp32 FMA chains (4 passes per step); mode 1 the matrix
 * waves only, 2 the vector waves only, 0 both. */
int tilemix_probe_coexec(int mode, int blocks, int iters, float* out, void* stream);

/* One 512-thread group per CU (128 KB of LDS): each wave issues `batch`
 * (1..16) direct 1 KB buffer->LDS copies from a `src_kb` KB device buffer,
 * waits for them, `iters` times. */
int tilemix_probe_copy(const void* src, int src_kb, int blocks, int iters, int batch, int* out, void* stream);

/* One 512-thread group per CU, each wave reading 16 KB of its own LDS region
 * per iteration with op 0 ds_read_b128 or op 1 ds_read_b64_tr_b16. */
int tilemix_probe_lds(int op, int blocks, int iters, int* out, void* stream);

/* Matrix skeleton of one prefill wave-tile per iteration, operands in
 * registers: 8 chained 32x32x32 int8 MFMAs, the scores converted to fp32,
 * `extra` (0, 64 or 128) further FMAs, packed to fp16, 16 32x32x16 f16
 * MFMAs (768 matrix cycles at the published peaks); `blocks` groups of 256
 * threads. */
int tilemix_probe_skeleton(int extra, int blocks, int iters, float* out, void* stream);

/* Shader clock: `blocks` groups of 256 threads run FMA chains for `iters`
 * steps; group 0 writes the shader-clock counter (s_memtime) before and
 * after into out[0], out[1] and the 100 MHz real-time counter into out[2],
 * out[3] (a device buffer of 4 int64). */
int tilemix_probe_clock(int blocks, int iters, long long* out, void* stream);

/* Reads the int8 k and v caches once (1,024 groups of 256 threads) in
 * pattern 0 (contiguous 64 KB per group), 1 (one 128-byte key row per lane),
 * 2 (8 lanes per key row) or 3 (as 2, the head fastest in launch order);
 * values are read 4 bytes per lane in patterns 1-3. */
int tilemix_probe_read(int pattern, const void* k, const void* v, int* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TILEMIX_PROBES_H */
