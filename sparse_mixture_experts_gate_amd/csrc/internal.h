// Host-side interface between the C-ABI layer (dsmoe_api.cpp) and the HIP
// kernel translation units. Internal to the library.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace dsmoe {

// ---- routing (router.hip) --------------------------------------------------
struct RouteParams {
  int64_t T;
  int E, K, G, M, topn;
  float eps;
};

// Split of the router's contraction for the bf16 path (partials are summed
// in a fixed order by the routing kernel). 1 for fp32 activations.
int router_splits(int64_t T, int d, int E, int act_dtype);
// fp32 activations: partial[0] = x . Wr^T with fp32 FMA accumulation.
hipError_t launch_router_f32(const float* x, const float* w, int64_t T, int d, int E, float* out,
                             hipStream_t s);
// bf16 activations: Wr split into bf16 hi + mid + lo (wsplit [E, 3d]), then
// `splits` partial sums [splits, T, E] of the exact products.
hipError_t launch_router_logits_bf16(const void* x, const float* w_router, int64_t T, int d, int E,
                                     int splits, uint16_t* wsplit, float* partial, hipStream_t s);
// Adds the split-K partials [splits, n] in split order into partial[0 .. n).
hipError_t launch_sum_partials(float* partial, int splits, int64_t n, hipStream_t s);
// Small batches (T <= kSmallRouterT, bf16 activations): fp32 logits straight
// from the fp32 router weights; also zeroes counts[E] and *near_tie.
constexpr int64_t kSmallRouterT = 32;
hipError_t launch_router_small(const void* x, const float* w, int64_t T, int d, int E, float* out,
                               int32_t* counts, int32_t* near_tie, hipStream_t s);
hipError_t launch_route(const float* partial, int splits, float* logits_out, const float* bias,
                        const RouteParams& p, int32_t* idx, float* gate, int32_t* counts,
                        int32_t* near_tie, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);

// ---- planning and permutation (permute.hip) --------------------------------
// Tile tables for the persistent grouped GEMMs: group g in [0, E) is routed
// expert g, group E the shared expert; tiles[g] = first tile of group g.
struct PlanParams {
  int64_t T;
  int E, K;
  int d, I, Is;
  int bm1, bnh1;  // GEMM1 rows per tile, intermediate columns per tile
  int bm2, bn2;   // GEMM2 rows per tile, output columns per tile
};
// counts != NULL: offsets_out = exclusive scan of counts. Else offsets_in is
// used. tiles1/tiles2 (may be NULL) receive the tile prefix of each group.
hipError_t launch_plan(const int32_t* counts, const int32_t* offsets_in, int32_t* offsets_out,
                       int32_t* tiles1, int32_t* tiles2, const PlanParams& p, hipStream_t s);
hipError_t launch_permute(const int32_t* idx, const int32_t* offsets, int64_t T, int K, int E,
                          int32_t* perm, int32_t* inv, hipStream_t s);
// dst[i, :] = src[perm[i], :] for i < n, rows of `row_bytes` bytes (multiple of
// 16); ids outside [0, n_src) give zero rows.
hipError_t launch_gather_rows(const void* src, int64_t n_src, const int32_t* perm, int64_t n,
                              int64_t row_bytes, void* dst, hipStream_t s);

// ---- grouped expert GEMMs ---------------------------------------------------
struct FfnArgs {
  const int32_t* offsets;  // [E+1]
  const int32_t* tiles1;   // [E+2]
  const int32_t* tiles2;   // [E+2]
  int64_t T, TK;
  int E, d, I, Is, ldh;
  // GEMM1 inputs
  const void* x;           // [T, d]; fp8: E4M3 codes
  const float* x_scale;    // fp8: [T, d/128]
  const int32_t* perm;     // gather rows of x for routed groups (NULL -> xperm)
  const void* xperm;       // [TK, d] contiguous routed rows (used when perm == NULL)
  const float* xperm_scale;
  float* xsT;              // fp8: activation scales [d/128, TK + T], k-block major: the
                           // routed rows in the permuted order, then the shared rows
  const void* w13;
  const void* ws13;
  const float* w13_scale;
  const float* ws13_scale;
  void* H;                 // [TK + T, ldh]
  float* H_scale;          // fp8: [ldh/128, TK + T], k-block major
  void* gu;                // training forward: pre-activations [TK + T, 2 ldh] bf16, or NULL
  void* h16;               // FP8 training forward: H [TK + T, ldh] in bf16, or NULL
  // GEMM2
  const void* w2;
  const void* ws2;
  const float* w2_scale;
  const float* ws2_scale;
  void* yperm;             // [TK, d]
  void* yshared;           // [T, d]
};

struct GemmTiling {
  int bm1, bnh1, bm2, bn2;
  int variant;  // kernel variant id, see gemm_bf16.hip / gemm_fp8.hip
};

GemmTiling choose_tiling(int64_t T, int K, int E, int w_dtype);
// fp32 tiles (gemm_f32.hip): 32 rows, 32 H columns / 64 output columns.
GemmTiling tiling_f32();
// FP8 tiles (gemm_fp8.hip), by the mean number of rows per expert.
GemmTiling choose_tiling_fp8(double rows_per_expert);
// `mid` (may be NULL) is recorded between the gate/up and the down GEMM.
hipError_t launch_ffn_bf16(const FfnArgs& a, const GemmTiling& t, hipStream_t s, hipEvent_t mid);
hipError_t launch_ffn_f32(const FfnArgs& a, hipStream_t s, hipEvent_t mid);
hipError_t launch_ffn_fp8(const FfnArgs& a, const GemmTiling& t, hipStream_t s, hipEvent_t mid);

// ---- backward (backward.hip), bf16 activations and weights ------------------
struct BwdArgs {
  const int32_t* offsets;  // [E+1]
  const int32_t* tiles;    // [E+2] tile prefix of the kernel's 128 x 256 tiles
  int64_t T, TK;
  int E, d, I, Is, ldh;
  const void* dyp;         // [TK, d] gated output gradients of the routed rows
  const void* dy;          // [T, d] output gradient (shared rows)
  const void* w2;          // [E, d, I] down projections, as in the forward
  const void* ws2;         // [d, Is]
  const void* w13;         // [E, 2I, d] gate/up projections, as in the forward
  const void* ws13;        // [2Is, d]
  const void* gu;          // [TK + T, 2 ldh] saved pre-activations
  void* dg;                // [TK + T, 2 ldh] [da | db] (OUT of dgrad2, IN of dgrad1)
  void* dap;               // [TK, d] OUT of dgrad1: input gradients of the routed rows
  void* das;               // [T, d] OUT of dgrad1: the shared expert's
};
struct WgradArgs {
  const int32_t* offsets;  // [E+1] segment starts of the routed rows
  int E;
  int64_t T;
  bool shared;             // a shared group (rows 0 .. T-1 of a_s, b_s) follows
  const void* a;           // routed rows [TK, lda] bf16 (row = token)
  const void* a_s;         // shared rows [T, lda_s]
  const void* b;           // routed rows [TK, ldb]
  const void* b_s;         // shared rows [T, ldb_s]
  int64_t lda, lda_s, ldb, ldb_s;
  int M, N;                // routed group output [M, N]: A columns x B columns
  int Ms, Ns;              // shared group output
  float* out;              // [E, M, N]
  float* out_s;            // [Ms, Ns]
};
hipError_t launch_bwd_gate(const void* dy, const void* yperm, const int32_t* idx,
                           const int32_t* inv, const float* gate, const float* logits, int64_t T,
                           int K, int E, int d, void* dyp, float* du, float* du_perm,
                           hipStream_t s);
hipError_t launch_bwd_combine(const void* dap, const void* das, const int32_t* inv,
                              const int32_t* idx, const float* du, const float* wr, int64_t T,
                              int K, int d, void* dx, hipStream_t s);
hipError_t launch_router_wgrad(const void* x, const int32_t* perm, const int32_t* offsets,
                               const float* du_perm, int E, int d, float* dwr, hipStream_t s);
hipError_t launch_dgrad2_bf16(const BwdArgs& a, hipStream_t s);
hipError_t launch_dgrad1_bf16(const BwdArgs& a, hipStream_t s);
hipError_t launch_wgrad_bf16(const WgradArgs& w, hipStream_t s);

// ---- FP8 backward (backward_fp8.hip) ----------------------------------------
// Input-gradient GEMMs on E5M2 gradients and the forward's E4M3 weights, read
// from transposed copies (rows along the contraction).
struct BwdFp8Args {
  const int32_t* offsets;     // [E+1]
  const int32_t* tiles_h;     // [E+2] 128 x 256 tiles over (rows, Ig)
  const int32_t* tiles_d;     // [E+2] 128 x 256 tiles over (rows, d)
  int64_t T, TK;
  int E, d, I, Is, ldh;
  const uint8_t* dyq;         // [TK, d] E5M2 gated output gradients, 1x128 scales dys
                              // (dys, dyss, dgs: k-block major, [blocks, rows])
  const float* dys;
  const uint8_t* dysq;        // [T, d] E5M2 output gradient (shared rows), scales dyss
  const float* dyss;
  const uint8_t* w2t;         // [E, I, d] E4M3 W2^T, scales [E, I/128, d/128]
  const float* w2t_scale;
  const uint8_t* ws2t;        // [Is, d], scales [Is/128, d/128]
  const float* ws2t_scale;
  const uint8_t* w13t;        // [E, d, 2I] E4M3 [W1; W3]^T, scales [E, d/128, 2I/128]
  const float* w13t_scale;
  const uint8_t* ws13t;       // [d, 2Is], scales [d/128, 2Is/128]
  const float* ws13t_scale;
  const uint16_t* gu;         // [TK + T, 2 ldh] saved pre-activations (bf16)
  uint16_t* dg;               // [TK + T, 2 ldh] OUT [da | db] bf16
  uint8_t* dgq;               // [TK + T, 2 ldh] OUT [da | db] E5M2
  float* dgs;                 // [TK + T, 2 ldh / 128] OUT its 1x128 scales
  uint16_t* dap;              // [TK, d] OUT input gradients of the routed rows
  uint16_t* das;              // [T, d] OUT the shared expert's
};
// Weight gradients out_g = A_g B_g^T from transposed 128x1-tile codes; qtiles
// [E+2] is the 128-row block prefix of the groups (routed, then shared).
struct WgradFp8Args {
  const int32_t* qtiles;
  int E;
  bool shared;
  const uint8_t* a;
  const float* as;
  const uint8_t* b;
  const float* bs;
  int M, N, Ms, Ns;
  float* out;                 // [E, M, N]
  float* out_s;               // [Ms, Ns]
};
// 128x1 quantization along each group's rows into the transposed layout:
// group g's C channels x npad_g tokens at byte C * 128 * qtiles[g] (the
// shared group after the routed ones, with Cs channels), scales
// [C, npad_g / 128] at float C * qtiles[g]. Routed rows: rows offsets[g] ..
// of src (row stride ld), or of src through perm; shared rows: rows of src_s.
struct QuantColsArgs {
  const int32_t* qtiles;
  const int32_t* offsets;
  int E;
  bool shared;
  int64_t T;
  const uint16_t* src;
  const int32_t* perm;
  int64_t ld;
  const uint16_t* src_s;
  int64_t ld_s;
  int C, Cs;
  uint8_t* q;
  float* scale;
};
hipError_t launch_dgrad2_fp8(const BwdFp8Args& a, hipStream_t s);
hipError_t launch_dgrad1_fp8(const BwdFp8Args& a, hipStream_t s);
// fa / fb: formats of A and B (0 = E4M3, 1 = E5M2); E5M2 x E4M3 only
hipError_t launch_wgrad_fp8(const WgradFp8Args& w, int fa, int fb, hipStream_t s);
// max_blocks: an upper bound of the groups' 128-row blocks (grid size)
hipError_t launch_quant_cols(const QuantColsArgs& q, int64_t max_blocks, int fmt, hipStream_t s);
// codes [n, rows, cols] -> [n, cols, rows]; block scales [n, rows/128, cols/128]
// -> [n, cols/128, rows/128]
hipError_t launch_transpose_fp8(const uint8_t* q, const float* scale, int64_t n_mats, int rows,
                                int cols, uint8_t* qt, float* scale_t, hipStream_t s);

// balance.hip: the sequence-level balance loss. part_p / part_c hold
// [n_seq * ceil(L / kBalanceChunk), E] partial sums, f - 1 [n_seq, E]; du16 [T, ldE] and
// duT16 [E, ldT] are bf16 copies of dloss/du (ldE, ldT multiples of 8).
constexpr int kBalanceChunk = 32;  // tokens per workgroup of the balance-loss kernels
hipError_t launch_seq_balance(const float* logits, const int32_t* idx, int64_t T, int E, int K,
                              int L, float alpha, float* part_p, int32_t* part_c, float* f,
                              float* loss, float* dlogits, uint16_t* du16, int ldE,
                              uint16_t* duT16, int64_t ldT, hipStream_t s);
// dst = bf16(src), n a multiple of 8.
hipError_t launch_to_bf16(const float* src, int64_t n, uint16_t* dst, hipStream_t s);
// off[g] = min(g * step, T), g = 0 .. G.
hipError_t launch_token_groups(int32_t* off, int G, int step, int64_t T, hipStream_t s);
// out = sum over g of part[g * n .. (g + 1) n), in g order; n a multiple of 4.
hipError_t launch_sum_groups(const float* part, int G, int64_t n, float* out, hipStream_t s);

// ---- elementwise (elementwise.hip) -----------------------------------------
hipError_t launch_combine(const void* yperm, const int32_t* inv, const float* gate,
                          const void* yshared, void* y, int64_t T, int K, int d, int io_dtype,
                          int out_dtype, hipStream_t s);
hipError_t launch_bias_update(const int32_t* counts, float gamma, float* bias, int E,
                              int64_t T, int K, hipStream_t s);
hipError_t launch_quant_blocks(const void* src, int src_dtype, int64_t n_mats, int rows,
                               int cols, uint8_t* q, float* scale, hipStream_t s);
// Row i of the output quantizes source row perm[i] (perm == NULL: row i);
// fmt 0 = E4M3, 1 = E5M2. Scales row-major [n, cols/128], or with kmajor
// k-block major [cols/128, n] (what the FP8 GEMMs read: a tile's row scales
// of one k block contiguous).
hipError_t launch_quant_rows(const void* src, int src_dtype, const int32_t* perm, int64_t n,
                             int cols, uint8_t* q, float* scale, hipStream_t s, int fmt = 0,
                             bool kmajor = false);

// number of compute units of the current device (cached per device)
int device_cu_count();

}  // namespace dsmoe
