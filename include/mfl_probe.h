/*
 * mfl_probe.h — test-only entry points of the MI355X fp16 GEMM library.
 *
 * They exist so tests can pin hardware facts the pages cannot: which lane and
 * register slot of a gfx950 matrix instruction holds which matrix element
 * (the role the SM80 thread/value tables play on the TiledMMA page
 * "读懂 CuTe 的 make_tiled_mma", section "从 C 的四个值开始读").
 */
#ifndef MFL_PROBE_H
#define MFL_PROBE_H

#include <stdint.h>

#include "mfl_gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* One wave (64 lanes) issues one matrix instruction `op` (numbering as
 * mfl_layout_mfma_tv).  Lane l takes A slots a_slots[l*VA .. l*VA+VA) and B
 * slots b_slots[l*VA ..] (fp16 bit patterns, VA = 8 for ops 0,1 and 4 for
 * ops 2,3) and accumulator inputs c_slots[l*VC .. +VC) (fp32, VC = 16 for the
 * 32x32 ops, 4 for the 16x16 ops); it writes its accumulator outputs to
 * d_out[l*VC .. +VC).  All four pointers are device memory sized 64*VA or
 * 64*VC elements.  Enqueued on `stream` (a hipStream_t).  Returns 0, -4 for
 * a bad op or NULL pointer, -5 on a launch error. */
int mfl_probe_mfma(int32_t op, const uint16_t* a_slots, const uint16_t* b_slots,
                   const float* c_slots, float* d_out, void* stream);

/* One wave fills a 4096-half LDS array from lds_in (device, 4096 fp16 bit
 * patterns) and issues one transposing LDS read (ds_read_b64_tr_b16) where
 * lane l addresses halves [lane_offsets[l], +4) (lane_offsets: host array of
 * 64 values, each a multiple of 4 in [0, 4092]); lane l writes the 4 halves it
 * receives to out[4l .. 4l+4) (device, 256 elements).  This pins the lane
 * regrouping the kernels rely on for an M-contiguous A operand (the role the
 * route page "ldmatrix 怎样对上 MMA 的寄存器" gives ldmatrix).  Returns 0,
 * -4 for a NULL pointer or an offset outside the rules, -5 on a launch error. */
int mfl_probe_lds_tr16(const int32_t* lane_offsets, const uint16_t* lds_in, uint16_t* out,
                       void* stream);

/* nblocks workgroups of 64 threads each write, to out[b] (device, nblocks
 * int32), the index 0..7 of the XCD (accelerator die) that ran workgroup b,
 * read from the XCC_ID hardware register.  This pins how workgroups are
 * dealt to the 8 XCDs, which the kernels' tile order assumes so that tiles
 * sharing operand rows share an XCD's L2 (a hardware fact the pages do not
 * cover).  Returns 0, -4 for nblocks outside [1, 65536] or a NULL pointer,
 * -5 on a launch error. */
int mfl_probe_xcc(int32_t nblocks, int32_t* out, void* stream);

/* Register dump of an LDS kernel (test-only): the kernel of configuration
 * `algo` (mfl_algo value, 2..10) with fetch policies fetch_a /
 * fetch_b (0 direct-to-LDS, 1 registers, 2 M-contiguous A transposed in
 * registers, 3 M-contiguous A direct-to-LDS) runs one K-step (K must equal
 * the configuration's BK) over M x N of whole tiles, A (M,K) K-contiguous
 * (or (K,M) M-contiguous for policies 2 and 3, lda >= M) and B (N,K) in
 * device memory with 16-byte aligned bases and lda, ldb multiples of 8.  In
 * place of the epilogue every thread of workgroup b writes, at out[(b *
 * threads + t) * words ..], its operand fragment registers (for each register
 * buffer, the RM A then the RN B fragments, 8 halves = 4 words each) and
 * then its RM x RN x NV fp32 accumulators: what the compiled fetch, LDS
 * layout, fragment reads and matrix instructions put in each register (the
 * per-thread coordinate dump of "cute(7) simple_gemm" §4, here for every
 * lane).  With out == NULL only *words_per_thread and *threads are set.
 * Returns 0, -4 for sizes, alignments or an out buffer outside these rules,
 * -6 when no dump instance exists for the combination, -5 on a launch
 * error.  Instances: every configuration with policies (0, 0); LDS_256 with
 * (1, 1), (2, 0), (3, 0); LDS_256_W4_16 with (1, 1), (3, 0). */
int mfl_probe_fragments(int32_t algo, int32_t fetch_a, int32_t fetch_b, int32_t M, int32_t N,
                        int32_t K, const uint16_t* A, int32_t lda, const uint16_t* B,
                        int32_t ldb, uint32_t* out, int64_t out_words, int32_t* words_per_thread,
                        int32_t* threads, void* stream);

/* gemm_tn (mfl_gemm.h: same arguments, checks and kernel choice) on a
 * test-only instance of the chosen LDS kernel that first fills its whole LDS
 * array with fp16 NaN: a fragment or epilogue read of any LDS location the
 * kernel did not write shows up in D.  Instances exist for C absent with fp32
 * D, fp16 C with fp16 D and fp32 C with fp32 D, on: LDS_128 with A/B fetch
 * direct-to-LDS or registers; LDS_256 with M-contiguous A direct-to-LDS and B
 * direct, or A transposed in registers and B in registers; LDS_128_W1 with A
 * direct and B in registers; LDS_SPLITK direct; LDS_256_W4_16 registers;
 * LDS_256_16 direct; LDS_128_16 M-contiguous A direct-to-LDS and B direct;
 * LDS_SPLITK_16 direct.
 * Returns gemm_tn's codes; MFL_E_ALGO_CASE (-6) where no instance exists for
 * the plan (force the kernel and fetch with the algo field). */
int mfl_probe_gemm_poisoned(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                            const void* B, int64_t ldb, const void* C, int64_t ldc, void* D,
                            int64_t ldd, gemm_dtypes_t dtypes, void* stream);

/* Measurement-only entry points: the rates the GEMM kernels are priced
 * against (a contraction is bound by the matrix cores; the pages' GEMMs, e.g.
 * "cute(7) simple_gemm" §10, only say the shared-memory version is faster).
 * Both write, for each workgroup b, clocks[4b .. 4b+4) = (shader-clock cycle
 * counter, 100 MHz real-time counter) before the timed loop and the same
 * after it (device memory, 4*nwg uint64), so the shader clock held during the
 * run is (cycles after - before) / (real time after - before) * 100 MHz.
 *
 * mfl_bench_mfma: nwg workgroups of 256 threads (4 waves, one per SIMD when
 * nwg = 256, the number of compute units); every wave fills 2 sets of operand
 * fragments from operands[0 .. n_operands) (device, fp16 bit patterns, read
 * cyclically: random or zero data is the caller's choice), then issues
 * iters x 32 v_mfma_f32_32x32x16_f16 (op 0; a 4 x 4 grid of 32x32 fp32
 * tiles, 2^20 FLOP per wave per iteration) or iters x 128
 * v_mfma_f32_16x16x32_f16 (op 1; 8 x 8 tiles of 16x16, 2^21 FLOP per wave per
 * iteration), and writes one float per
 * thread to sink (device, 256*nwg floats) so the work is not removed.
 * Returns 0, -4 for a bad op, size or NULL pointer, -5 on a launch error.
 *
 * mfl_bench_lds_read: nwg workgroups of `threads` threads (a multiple of 64,
 * at most 1024), each with 96 KB of LDS (one workgroup per compute unit);
 * every wave issues iters x 16 ds_read_b128, each covering 1 KB contiguously
 * (64 lanes x 16 bytes, every bank once per 16-lane pass): 16 KB per wave per
 * iteration, in groups of `depth` reads (1, 4, 8 or 16) that are all issued
 * before the first is consumed, so `depth` reads are in flight per wave.
 * sink: device, nwg uint32.  Returns 0, -4 for a bad size, depth or NULL
 * pointer, -5 on a launch error. */
int mfl_bench_mfma(int32_t op, const uint16_t* operands, int32_t n_operands, int32_t iters,
                   int32_t nwg, float* sink, uint64_t* clocks, void* stream);
int mfl_bench_lds_read(int32_t threads, int32_t iters, int32_t nwg, int32_t depth,
                       uint32_t* sink, uint64_t* clocks, void* stream);

/* Direct-to-LDS fetch rate: nwg workgroups of `threads` threads (a multiple
 * of 64, at most 1024), each with 96 KB of LDS (one workgroup per compute
 * unit); workgroup g re-reads bytes [g * 65536, (g + 1) * 65536) of buf
 * (device, nwg * 65536 bytes, contents ignored; the region stays in L2) in
 * 1 KB runs with global_load_lds_dwordx4, every wave issuing iters x `depth`
 * instructions (depth 4, 12 or 24) and waiting for each batch of `depth`
 * before the next: iters x depth KB per wave.  sink (device, nwg uint32) and
 * clocks (device, 4 * nwg uint64: cycle and real-time counters before and
 * after the loop, per workgroup) as in mfl_bench_lds_read.  Returns 0, -4
 * for a bad size, depth or NULL pointer, -5 on a launch error. */
int mfl_bench_dma_rate(int32_t threads, int32_t iters, int32_t nwg, int32_t depth,
                       const uint8_t* buf, uint32_t* sink, uint64_t* clocks, void* stream);

/* The rate of the real-time counter the three entry points above record, in
 * kHz, for the current device (*khz, host memory).  Returns 0, -4 for a NULL
 * pointer, -5 when the runtime does not report it. */
int mfl_wall_clock_khz(int32_t* khz);

/* Phase timing of the back-to-back GEMM of mfl_chain.h (the Tensor Core
 * page "CuTe Layout 到 Tensor Core", §17: the accumulator of one MMA read as
 * the next MMA's operand).  Same arguments, checks, result in D and error
 * codes as gemm_tn_chain, for the configuration K = 128, N2 > 64, fp16 D,
 * direct-to-LDS staging (else -4); the kernel is a separate instance in which
 * lane 0 of every wave also records the low 32 bits of the shader-clock
 * counter (s_memtime) at fixed points.  stamps: device memory of 8 x 8 x 260
 * uint32, written for workgroups 0..7 (fewer if the grid is smaller), wave w
 * (0..7) of workgroup g at [(8 g + w) * 260 + q]: for iteration c < 64 of the N1
 * loop, q = 4c at its start, 4c + 1 before the wave waits for its fetch of
 * the next slot, 4c + 2 before the workgroup barrier, 4c + 3 after it
 * (the last iteration records only 4c); q = 256 kernel start, 257 after the
 * loop, 258 after the epilogue.  Stamps of one wave come from one counter.
 * The kernel keeps the readings in registers until its end (no LDS traffic,
 * no added waits): they cost a few scalar and vector instructions per
 * iteration.  NULL stamps: -3. */
int mfl_probe_chain_phases(int64_t batch, int64_t M, int64_t N1, int64_t N2, int64_t K,
                           const void* A, int64_t lda, int64_t stride_a, const void* B,
                           int64_t ldb, int64_t stride_b, const void* W, int64_t ldw,
                           int64_t stride_w, void* D, int64_t ldd, int64_t stride_d,
                           int32_t d_dtype, uint32_t* stamps, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MFL_PROBE_H */
