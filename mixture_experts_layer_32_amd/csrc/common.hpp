// Device-side building blocks shared by the LatentMoE kernels (gfx950, wave64).
//
// Data movement is done in 16-byte "chunks" (one dwordx4 per lane, type u32x4).  A chunk
// holds 8 bf16, 4 fp32 or 16 fp8 values.  MFMA operands are consumed one
// chunk per lane: for v_mfma_f32_16x16x32_bf16 the 64 lanes form 4 groups of
// 16; lane l supplies row (l % 16) of its operand and the 8 reduction indices
// of its group (l / 16).  Only the pairing of A and B lanes matters for the
// reduction, so any fixed assignment of reduction indices to (group, chunk)
// that both operands share gives the same sum; the kernels use that freedom
// to make each lane's loads contiguous.
//
// Result layout of a 16x16 fp32 accumulator (4 VGPRs): lane l, element v
// holds C[row = 4 * (l / 16) + v][col = l % 16].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace lmoe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// One 16-byte chunk.  A native vector type (not HIP's uint4 struct) so that
// selects and copies stay in registers.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, WGs dispatched round-robin

// A 16-byte zero chunk in global memory (one per translation unit).  Loads of
// padding rows and of chunks past the end of K read it: selecting the ADDRESS
// keeps the loaded value usable as is, whereas selecting between the loaded
// value and zero would force a wait on the load right where it is issued.
static __device__ __attribute__((aligned(16))) uint32_t g_zero_chunk[4] = {0u, 0u, 0u, 0u};

__device__ __forceinline__ u32x4 load_chunk(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Raw (byte-addressed, stride 0) buffer resource: 64-bit base in SGPRs, a
// byte range, and dword 3 = DATA_FORMAT 32-bit (value 4 in bits 15..18).
// A buffer load whose offset lies past the range returns zeros, so loads
// need only a 32-bit per-lane offset and padding costs no select on data.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
constexpr uint32_t kOutOfRange = 0x80000000u;  // an offset that always reads as zero

__device__ __forceinline__ BufRsrc make_rsrc(const void* base, uint64_t bytes) {
  const int n = bytes >= 0x80000000ull ? 0x7fffffff : static_cast<int>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

// Cache policy of a buffer load: 0 = default, kCpolNonTemporal = data read
// once (expert weights): streamed without displacing reused lines.
constexpr int kCpolDefault = 0;
constexpr int kCpolNonTemporal = 2;

template <int CPOL = kCpolDefault>
__device__ __forceinline__ u32x4 buffer_load_chunk(BufRsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                       r, static_cast<int>(voff), static_cast<int>(soff), CPOL));
}

// One 16-byte chunk per lane straight from global memory into LDS: lane i of
// the wave writes bytes [16 i, 16 i + 16) after the wave-uniform LDS byte
// address `lds`; an out-of-range offset writes zeros.  The load counts in
// vmcnt like any vector load, and nothing orders later LDS reads after it
// except an explicit wait (wait_vmcnt_lgkm0) and, across waves, a barrier.
// Written as inline asm: the compiler's own form of this load makes it wait
// for every LDS-mode load in flight before any later LDS read it cannot
// prove disjoint, which collapses a ring of stage buffers to one stage.  The
// memory clobber keeps the load in program order against LDS reads; M0
// carries the LDS address (an operand: the compiler sets it).
__device__ __forceinline__ void dma16_to_lds(BufRsrc r, uint32_t lds, uint32_t voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "{m0}"(lds)
               : "memory");
}

// LDS byte address of a shared-memory pointer, as a wave-uniform value
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p)));
}

__device__ __forceinline__ void buffer_load_chunk_lds(BufRsrc r, u32x4* lds, uint32_t voff) {
  dma16_to_lds(r, lds_addr(lds), voff);
}

// LDS-only barrier: this wave's LDS operations are complete and every wave
// of the workgroup has arrived.  Global loads and stores in flight are not
// waited for (an LDS-scoped fence around s_barrier).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (expcnt untouched).  gfx9 encoding: vmcnt
// bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN): the gfx950
// conversion instruction v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// two fp32 -> two bf16 in one dword (lo in bits 0..15), one instruction
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Four OCP E4M3 bytes -> four bf16 (packed in two dwords).  Every E4M3
// value is exactly representable in bf16, so taking the upper half of the
// fp32 produced by the hardware conversion is exact.
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t q) {
  f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(q), false);
  f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(q), true);
  uint2 r;
  r.x = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xffff0000u);
  r.y = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xffff0000u);
  return r;
}

// MXFP4 weights (OCP MX: FP4 E2M1 elements, element 2j in the low nibble of
// byte j, one E8M0 power-of-two scale per 32 elements).  The storage type of
// a pair of elements:
struct fp4x2_t {
  uint8_t v;
};

// E8M0 scale byte -> fp32 2^(e - 127) as the OCP MX format defines it: e = 0
// is the subnormal 2^-127 (fp32 bits 0x00400000) and e = 0xFF is NaN
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  const uint32_t b = e == 0u ? 0x00400000u : (e == 0xFFu ? 0x7fc00000u : e << 23);
  return __uint_as_float(b);
}

// Eight E2M1 elements (one dword) times the block scale -> eight bf16 (one
// 16-byte MFMA operand), with the gfx950 scaled conversion
// v_cvt_scalef32_pk_bf16_fp4 (byte b -> elements 2b, 2b + 1; exact: an E2M1
// value times a power of two is a bf16 value)
__device__ __forceinline__ u32x4 fp4x8_to_bf16x8(uint32_t q, float scale) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 0)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 1)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 2)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 3))};
}

// one byte through a buffer resource (out-of-range offsets read 0)
__device__ __forceinline__ uint32_t buffer_load_byte(BufRsrc r, uint32_t voff) {
  return static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b8(r, static_cast<int>(voff), 0, 0));
}

// 16 E4M3 bytes (one chunk) -> 16 bf16 (two chunks).
__device__ __forceinline__ void fp8_chunk_to_bf16(u32x4 q, u32x4& lo, u32x4& hi) {
  uint2 a = fp8x4_to_bf16x4(q.x), b = fp8x4_to_bf16x4(q.y);
  uint2 c = fp8x4_to_bf16x4(q.z), d = fp8x4_to_bf16x4(q.w);
  lo = u32x4{a.x, a.y, b.x, b.y};
  hi = u32x4{c.x, c.y, d.x, d.y};
}

// ---------------------------------------------------------------- MFMA chunks
//
// Each MFMA flavour describes, for the tiled GEMM: its output block (BLK x
// BLK), how many 16-byte chunks of K one MFMA consumes per row (CPS), which
// fragment row and which of those chunks a lane supplies, and where
// accumulator element v of a lane sits in the output block.

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// v_mfma_f32_16x16x32_bf16: acc += A_chunk x B_chunk over the 8 reduction
// indices of each of the 4 lane groups (lane l: row l % 16, group l / 16).
struct MmaBf16 {
  static constexpr int kElemBytes = 2;
  static constexpr int BLK = 16, CPS = 4, NV = 4;
  typedef f32x4_t Acc;
  __device__ __forceinline__ static void mma(f32x4_t& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
  __device__ __forceinline__ static int frag_row(int lane) { return lane & 15; }
  __device__ __forceinline__ static int frag_chunk(int lane) { return lane >> 4; }
  __device__ __forceinline__ static int out_row(int lane, int v) { return 4 * (lane >> 4) + v; }
  __device__ __forceinline__ static int out_col(int lane) { return lane & 15; }
  // operands swapped (B fragment first): the block is computed transposed,
  // so lane l holds row l % 16, columns 4 (l / 16) + 0..3
  __device__ __forceinline__ static int t_row(int lane) { return lane & 15; }
  __device__ __forceinline__ static int t_col(int lane, int) { return 4 * (lane >> 4); }
};

// v_mfma_f32_32x32x16_bf16: lane l supplies row l % 32 and the 8 reduction
// indices (one chunk) of half l / 32: two chunks of K per MFMA.
// Result: lane l, element v holds C[8 (v / 4) + 4 (l / 32) + v % 4][l % 32].
// A 32x32 block is twice the work per operand byte of a 16x16 one, and
// issues back to back with only a few independent accumulators.
struct MmaBf16x32 {
  static constexpr int kElemBytes = 2;
  static constexpr int BLK = 32, CPS = 2, NV = 16;
  typedef f32x16_t Acc;
  __device__ __forceinline__ static void mma(f32x16_t& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
  __device__ __forceinline__ static int frag_row(int lane) { return lane & 31; }
  __device__ __forceinline__ static int frag_chunk(int lane) { return lane >> 5; }
  __device__ __forceinline__ static int out_row(int lane, int v) {
    return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
  }
  __device__ __forceinline__ static int out_col(int lane) { return lane & 31; }
  // operands swapped: lane l holds row l % 32, columns 8 g + 4 (l / 32) + 0..3
  // in elements 4 g .. 4 g + 3
  __device__ __forceinline__ static int t_row(int lane) { return lane & 31; }
  __device__ __forceinline__ static int t_col(int lane, int g) { return 8 * g + 4 * (lane >> 5); }
};

// fp32: a chunk is 4 values; element s of every group's chunk feeds one
// v_mfma_f32_16x16x4_f32 (group g supplies reduction index g of that MFMA).
struct MmaF32 {
  static constexpr int kElemBytes = 4;
  static constexpr int BLK = 16, CPS = 4, NV = 4;
  typedef f32x4_t Acc;
  __device__ __forceinline__ static void mma(f32x4_t& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[0]), __uint_as_float(b[0]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[1]), __uint_as_float(b[1]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[2]), __uint_as_float(b[2]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[3]), __uint_as_float(b[3]), acc, 0, 0, 0);
  }
  __device__ __forceinline__ static int frag_row(int lane) { return lane & 15; }
  __device__ __forceinline__ static int frag_chunk(int lane) { return lane >> 4; }
  __device__ __forceinline__ static int out_row(int lane, int v) { return 4 * (lane >> 4) + v; }
  __device__ __forceinline__ static int out_col(int lane) { return lane & 15; }
  // operands swapped (B fragment first): the block is computed transposed,
  // so lane l holds row l % 16, columns 4 (l / 16) + 0..3
  __device__ __forceinline__ static int t_row(int lane) { return lane & 15; }
  __device__ __forceinline__ static int t_col(int lane, int) { return 4 * (lane >> 4); }
};

// ---------------------------------------------------------------- epilogue

// SwiGLU output from an up-projection value and its gate: up * SiLU(gate),
// SiLU(b) = b / (1 + e^-b), with the hardware exp2 and reciprocal (about 1
// ulp each; e^-b as 2^(-b log2 e), whose argument rounding adds a relative
// error near |b| 2^-24): all far below the bf16 rounding of the output and
// the 1e-4 relative bound of an fp32 output
__device__ __forceinline__ float swiglu(float up, float gate) {
  const float e = __builtin_amdgcn_exp2f(gate * -1.4426950408889634f);
  return up * gate * __builtin_amdgcn_rcpf(1.f + e);
}

template <int ACT>
__device__ __forceinline__ float apply_act(float v) {
  if constexpr (ACT == kActSqRelu) {
    // max(v, 0) on the bit pattern: a set sign bit is a negative integer,
    // so negative inputs (and -0) become +0 in one integer max
    const float r = __builtin_bit_cast(float, max(__builtin_bit_cast(int, v), 0));
    return r * r;
  } else {
    return v;
  }
}

template <typename TOut>
__device__ __forceinline__ void store_elem(TOut* p, float v);
template <>
__device__ __forceinline__ void store_elem<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_elem<uint16_t>(uint16_t* p, float v) { *p = f32_to_bf16(v); }

// ---------------------------------------------------------------- scheduling

// Work item for workgroup `b` of a grid of `grid` WGs covering `total` items,
// such that each XCD (b % 8) receives one contiguous range of items: items
// that share operands (the N tiles of one M tile, the tiles of one expert)
// then run on the same XCD and share its L2.  Returns -1 for idle WGs.
// Requires grid to be a multiple of 8 and >= total rounded up to 8.
__device__ __forceinline__ int xcd_contiguous_item(int b, int grid, int total) {
  const int per = grid / kNumXcd;
  const int xcd = b % kNumXcd;
  const int local = b / kNumXcd;
  const int per_used = (total + kNumXcd - 1) / kNumXcd;
  if (local >= per_used) return -1;
  const int item = xcd * per_used + local;
  (void)per;
  return item < total ? item : -1;
}

// ---------------------------------------------------------------- wave reductions
//
// DPP (data-parallel primitives) reductions over a full wave of 64 lanes:
// quad permutations and half-row / row mirrors combine the 16 lanes of each
// row, then the GFX9 row broadcasts carry row 0 into row 1, row 2 into row 3
// and lane 31 into rows 2-3, so lane 63 ends with the reduction of all lanes.
// Every lane must be active.  The result is read back from lane 63.
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  // rows outside ROW_MASK keep their own value
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v),
                                                           CTRL, ROW_MASK, 0xF, false));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppQuadXor1>(v));
  v = max(v, dpp_u32<kDppQuadXor2>(v));
  v = max(v, dpp_u32<kDppRowHalfMirror>(v));
  v = max(v, dpp_u32<kDppRowMirror>(v));
  v = max(v, dpp_u32<kDppRowBcast15, 0xA>(v));
  v = max(v, dpp_u32<kDppRowBcast31, 0xC>(v));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<kDppQuadXor1>(v));
  v = min(v, dpp_u32<kDppQuadXor2>(v));
  v = min(v, dpp_u32<kDppRowHalfMirror>(v));
  v = min(v, dpp_u32<kDppRowMirror>(v));
  v = min(v, dpp_u32<kDppRowBcast15, 0xA>(v));
  v = min(v, dpp_u32<kDppRowBcast31, 0xC>(v));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

__device__ __forceinline__ float wave_sum(float v) {
  v +=__uint_as_float(dpp_u32<kDppQuadXor1>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppQuadXor2>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppRowHalfMirror>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppRowMirror>(__float_as_uint(v)));
  // row broadcasts add into the receiving rows only; other rows add zero
  v += __uint_as_float(__builtin_amdgcn_update_dpp(0, static_cast<int>(__float_as_uint(v)),
                                                   kDppRowBcast15, 0xA, 0xF, false));
  v += __uint_as_float(__builtin_amdgcn_update_dpp(0, static_cast<int>(__float_as_uint(v)),
                                                   kDppRowBcast31, 0xC, 0xF, false));
  return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(__float_as_uint(v)), 63)));
}

}  // namespace lmoe
