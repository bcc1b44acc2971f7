// Host-side launch interface of the LatentMoE kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmoe {

enum class Dt : int { F32 = 0, BF16 = 1, FP8 = 2, MXFP4 = 3 };
// kActSwiGlu: the B rows are interleaved pairs (row 2i the up projection
// W_FC1 row i, row 2i + 1 the gate W_gate row i) and output column i is
// C[2i] * SiLU(C[2i + 1]): the output is N / 2 wide.
enum ActKind : int { kActNone = 0, kActSqRelu = 1, kActSwiGlu = 2 };

// C = act(scale . (A x B^T)), all operands K-contiguous ("[rows][K]").
// Dense: one group of M rows.  Grouped: group g owns logical rows
// [g_off[g], g_off[g+1]) and weight matrix B + g * b_gstride; g_tiles is
// the exclusive prefix of ceil(rows_g / BM) computed on the device.
struct GemmArgs {
  const void* A = nullptr;
  int64_t lda = 0;                 // elements
  const int32_t* a_rows = nullptr; // optional gather: A row of logical row r is a_rows[r]
  int a_nrows = 0;                 // rows of A (bounds the gathered reads)
  const void* B = nullptr;
  int64_t ldb = 0;                 // elements
  int64_t b_gstride = 0;           // elements between group weight matrices
  const float* b_scale = nullptr;  // per output column (row of B) scale, fp8 weights
  int64_t s_gstride = 0;
  void* C = nullptr;
  int64_t ldc = 0;
  int M = 0, N = 0, K = 0;
  const int32_t* g_off = nullptr;  // [G+1], nullptr = dense
  const int32_t* g_tiles = nullptr;// [G+1] (tiled kernel only)
  int G = 1;
  int max_rows = 0;                // grouped: upper bound of the total rows (sizes the grid)
  int act = 0;                     // ActKind
  // dense only: output columns n >= N0 take row n - N0 of B2 instead of B
  // (two weight matrices over the same A in one launch; N0 a multiple of
  // the column tile, split-K partial output only)
  const void* B2 = nullptr;
  int N0 = 0;
  // dense only: fp32 residual added to the output before its one rounding,
  // C[r][c] = act(...) + R[r * ldr + c] (N, ldr multiples of 4, R 16-byte aligned)
  const float* R = nullptr;
  int64_t ldr = 0;
  // MXFP4 weights (streaming kernel): B holds E2M1 pairs (ldb, b_gstride in
  // bytes), b_mx the E8M0 scales of each row's blocks of 32 (mx_ld bytes per
  // row, mx_gstride per group)
  const uint8_t* b_mx = nullptr;
  int64_t mx_gstride = 0, mx_ld = 0;
  // streaming kernel, sparse batches: g_active[0 .. g_tiles[G]) lists the
  // groups with rows, and only those are visited
  const int32_t* g_active = nullptr;
  // grouped kernel: A (gathered or not) or C stored in blocks of 32
  // columns, block b holding columns 32 b .. 32 b + 31 of rows 0 .. kblock - 1
  // (64 bytes per row, lda / ldc unused); 0 = row-major
  int a_kblock = 0;
  int c_kblock = 0;
  // grouped kernels: B in bands of rows, a band as its 64-byte column blocks
  // one after another (launch_pack_bands; 256-row bands for the bf16
  // grouped kernel, 16-row bands for the fp8 one); ldb == K
  int b_bands = 0;
  // dense grouped kernel only (no g_off, no activation): a second copy of C
  // in 32-column blocks over the M rows (block b: columns 32 b .. 32 b + 31
  // of rows 0 .. M - 1, 64 bytes per row), written beside the row-major C
  void* C2 = nullptr;
};

// LDS-tiled MFMA GEMM.  tile: 0 = 128x128, 1 = 64x64, 2 = 256x256,
// 3 = 128x256 block tile.
// splits > 1 (dense only): K is split and fp32 partial tiles go to `partial`
// ([splits][M][N] floats) before a fixed-order reduction (split 0 + split 1
// + ...), which a second kernel performs unless reduce is false: then the
// consumer adds the partials itself, in the same order.
hipError_t launch_gemm_tiled(const GemmArgs& a, Dt a_dt, Dt out_dt, int tile, hipStream_t s,
                             int splits = 1, float* partial = nullptr, bool reduce = true);
int tiled_block_m(int tile);
// Grouped GEMM with OCP E4M3 weights (b_scale: one fp32 scale per weight
// row), bf16 activations and output: 96-row tiles (g_tiles counts them),
// weights streamed into registers.  Needs N and K multiples of 16, at most
// 2048 groups.
bool gemm_fp8w_fits(int N, int K, int G);
// b_bands: B in 16-row bands of 64-byte blocks (launch_pack_bands), K a
// multiple of 64
hipError_t launch_gemm_fp8w(const GemmArgs& a, hipStream_t s);
int fp8w_block_m();

// Grouped GEMM for experts with many rows (prefill), bf16 operands and
// output: a persistent grid walks (expert, row tile, 256-column tile) items;
// an expert's last row tile is 256, 128 or 64 rows high.  Needs N a multiple
// of 256, K of 32, at most 2048 groups; g_tiles is not read.  Without g_off
// it is a dense GEMM: one group (G = 1) of M rows, A not gathered.
bool gemm_grouped_fits(int N, int K, int G);
// Band layout of G row-major matrices of N rows x row_bytes: bands of
// band_rows rows, a band as its 64-byte column blocks one after another (a
// block = band_rows rows x 64 bytes).  gemm_grouped's b_bands: bf16, 256-row
// bands; gemm_fp8w's: E4M3, 16-row bands.  N a multiple of band_rows,
// row_bytes of 64.
hipError_t launch_pack_bands(const void* src, void* dst, int G, int N, int row_bytes, int band_rows,
                             hipStream_t s);
hipError_t launch_gemm_grouped(const GemmArgs& a, hipStream_t s);

// Compute units of the current device (queried once per device; 256 on
// MI355X), for persistent grids.
int device_compute_units();

// Weight-streaming grouped GEMM for few rows per group (decode regime), bf16,
// fp8 (per-row scales) or MXFP4 (block scales, K a multiple of 32) weights:
// every group's weight matrix is streamed from HBM once per pass of up to
// mrows_max rows.  mb_max: 4 or 8 (rows per pass = 16 * mb_max).
hipError_t launch_gemm_stream(const GemmArgs& a, Dt a_dt, Dt w_dt, Dt out_dt, int mb_max,
                              hipStream_t s);

// Fused expert FFN for few rows per expert (decode regime), bf16:
// Y[r] = sqrelu(A[a_rows[r]] W1_g^T) W2_g^T for the rows r of each group g,
// the hidden row kept on chip.  One resident workgroup per compute unit
// takes whole experts; an expert with more than ffn_stream_rows() rows is
// processed in several passes (its weights streamed once per pass).
struct FfnArgs {
  const void* A = nullptr;          // token rows [a_nrows][lda] (u)
  int64_t lda = 0;
  const int32_t* a_rows = nullptr;  // A row of grouped row r (token_of)
  int a_nrows = 0;
  const void* W1 = nullptr;         // [G][m][l]
  const void* W2 = nullptr;         // [G][l][m]
  void* Y = nullptr;                // [rows][ldy]
  int64_t ldy = 0;
  const int32_t* g_off = nullptr;   // [G+1] first grouped row of each group
  int G = 0;
  int l = 0, m = 0;
  int act = kActSqRelu;             // or kActSwiGlu: W1 is [G][2m][l], rows interleaved
  // MXFP4 weights: W1, W2 hold E2M1 pairs, W1_mx [G][m or 2m][l/32] and
  // W2_mx [G][l][m/32] their E8M0 block scales (l, m multiples of 32)
  const uint8_t* W1_mx = nullptr;
  const uint8_t* W2_mx = nullptr;
};
// Whether the fused kernel takes this shape: the hidden rows fit in LDS,
// and each weight array of all G experts stays below 2 GiB.
bool ffn_stream_fits(int G, int l, int m, bool glu, bool fp4);
int ffn_stream_rows();
hipError_t launch_ffn_stream(const FfnArgs& a, hipStream_t s);

// Routing.
// Top-k selection and gates, one wave per token.  The logits may arrive as
// the split-K partials of the router GEMM ([lsplits][T][N]), added here in
// split order; the kernel can also finish the down-projection (its split-K
// partials [usplits][T][l] added the same way, written to u), which no
// earlier stage needs when the router reads x.
struct TopkArgs {
  const float* logits = nullptr;  // split z, token t, expert e at z*logits_sstride + t*logits_ld + e
  int64_t logits_ld = 0, logits_sstride = 0;
  int lsplits = 1;
  float* logits_out = nullptr;    // reduced logits [T][N] (before the bias), or nullptr
  const float* bias = nullptr;    // [N] or nullptr
  int T = 0, N = 0, K = 0, gating = 0;
  int32_t* idx = nullptr;         // [T][K]
  float* gate = nullptr;          // [T][K]
  const float* u_part = nullptr;  // split z, token t, column c at z*u_sstride + t*u_ld + c
  int64_t u_ld = 0, u_sstride = 0;
  int usplits = 1, l = 0;
  void* u = nullptr;              // [T][l], bf16 (u_bf16) or fp32
  int u_bf16 = 1;
};
hipError_t launch_topk_gate(const TopkArgs& a, hipStream_t s);
hipError_t launch_route_masks(const int32_t* idx, int T, int N, int K, uint64_t* masks,
                              hipStream_t s);
// active (optional, with tile_m = kActiveTile): the ids of the experts with
// copies in ascending order, [tiles[N]] of them (tiles[e] is then the number
// of such experts before e)
constexpr int kActiveTile = 1 << 30;
hipError_t launch_route_scan(const uint64_t* masks, int nblk, int N, int tile_m, int32_t* counts,
                             int32_t* offsets, int32_t* base, int32_t* tiles, hipStream_t s,
                             int32_t* active = nullptr);
hipError_t launch_route_assign(const int32_t* idx, const uint64_t* masks, const int32_t* base,
                               const int32_t* offsets, int T, int N, int K, int32_t* slot_of,
                               int32_t* token_of, hipStream_t s);
// masks + scan + assign in one launch, when the per-block masks fit
// in LDS (ceil(T/64) * N small): one launch instead of three.
bool route_small_fits(int T, int N, int K);
hipError_t launch_route_small(const int32_t* idx, int T, int N, int K, int tile_m, int32_t* counts,
                              int32_t* offsets, int32_t* tiles, int32_t* slot_of,
                              int32_t* token_of, hipStream_t s, int32_t* active = nullptr);
// v[t] = sum_j gate[t][j] * Y[slot_of[t][j]] (+ R[t], fp32 [T][l], when R is given)
hipError_t launch_combine(const void* Y, const int32_t* slot_of, const float* gate, int T, int K,
                          int l, Dt dt, const float* R, void* v, hipStream_t s);

constexpr int kRouteBlock = 64;  // tokens per routing block (one 64-bit mask per expert)

}  // namespace lmoe
