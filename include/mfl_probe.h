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

#ifdef __cplusplus
}
#endif
#endif /* MFL_PROBE_H */
