// ragged_mm on CDNA4 matrix cores: one 128x128 output tile of a grouped
// (per-expert) matrix product, computed by one 256-thread workgroup.
//
// The Latch pages ("What Latch does", step 1 and step 3) name ragged_mm as the
// grouped expert product whose bucket sizes change every update, with
// derivative rules for its backward.  Here each tile is C[m,n] = sum_k A[m,k]
// B[k,n] with fp32 accumulation on MFMA (bf16: v_mfma_f32_32x32x16_bf16; fp32
// mode: v_mfma_f32_32x32x2_f32).
//
// Operands are staged through LDS in a [row][k] layout (k contiguous, 128
// bytes of k per row and stage, rows padded to 144 bytes).  An operand whose
// source rows run along k ("direct": activations in the forward products,
// weights read as W^T) is copied 16 bytes at a time.  An operand whose source
// rows run along m or n ("transposed": weights read as W, and both operands of
// the weight-gradient products, where k runs over the routed tokens) is loaded
// as 4 k-rows x 16 bytes per thread and transposed in registers before the
// LDS write.  Row indices may go through a map (the dispatch gather: row =
// perm[p] / k), so no gathered copy of the tokens is ever materialised.
// Two LDS stages: the global loads of k-tile i+1 are in flight while the
// matrix cores work on k-tile i.
#pragma once

#include "device_common.h"

namespace moe {
namespace gemm {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int KBYTES = 128;              // bytes of k per LDS row per stage
constexpr int ROW = 144;                 // padded LDS row stride (bytes)
constexpr int A_BYTES = BM * ROW;
constexpr int B_BYTES = BN * ROW;
constexpr int STAGE = A_BYTES + B_BYTES;
constexpr int LDS_BYTES = 2 * STAGE;     // 73,728 bytes

// One operand of a tile.
//   direct:     logical row r (0..127) -> source row map(p0 + r), k runs along it;
//               rows r >= nrows and k >= lim read as zero.
//   transposed: logical k-row kk -> source row map(p0 + kk), the tile's m/n
//               columns mn0.. run along it; k-rows kk >= nrows and columns
//               >= lim read as zero.
struct Operand {
  const char* base;   // bytes
  long ld;            // source row stride in elements
  const int* map;     // optional row map (NULL = identity)
  int div;            // row = map[p] / div
  int p0;
  int nrows;
  int lim;
  int mn0;
};

__device__ __forceinline__ long map_row(const Operand& o, int p) {
  return o.map ? (long)(o.map[p] / o.div) : (long)p;
}

template <typename T>
struct Loader {
  static constexpr int VEC = 16 / (int)sizeof(T);    // elements per 16 bytes
  static constexpr int BKE = KBYTES / (int)sizeof(T);  // k elements per stage
  static constexpr int MBC = 128 / VEC;               // 16-byte column groups per tile row

  // direct operands: source byte offsets of this thread's 4 rows (or -1)
  long rowoff[4];

  __device__ __forceinline__ void init_direct(const Operand& o) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      rowoff[i] = (r < o.nrows) ? map_row(o, o.p0 + r) * o.ld * (long)sizeof(T) : -1;
    }
  }

  __device__ __forceinline__ void load_direct(const Operand& o, int kt, uint4 (&v)[4]) const {
    const int c = threadIdx.x & 7;
    const int col = kt * BKE + c * VEC;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (rowoff[i] >= 0 && col < o.lim)
        x = *reinterpret_cast<const uint4*>(o.base + rowoff[i] + (long)col * (long)sizeof(T));
      v[i] = x;
    }
  }

  __device__ __forceinline__ static void load_trans(const Operand& o, int kt, uint4 (&v)[4]) {
    const int tid = threadIdx.x;
    const int mb = tid % MBC, kb = tid / MBC;
    const int mn = o.mn0 + mb * VEC;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = kt * BKE + kb * 4 + i;
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (kk < o.nrows && mn < o.lim) {
        const long row = map_row(o, o.p0 + kk);
        x = *reinterpret_cast<const uint4*>(o.base + (row * o.ld + mn) * (long)sizeof(T));
      }
      v[i] = x;
    }
  }

  __device__ __forceinline__ static void store_direct(char* lds, const uint4 (&v)[4]) {
    const int tid = threadIdx.x;
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      *reinterpret_cast<uint4*>(lds + r * ROW + c * 16) = v[i];
    }
  }

  __device__ __forceinline__ static uint32_t half16(const uint4& u, int j) {
    const uint32_t w = (j >> 1) == 0 ? u.x : (j >> 1) == 1 ? u.y : (j >> 1) == 2 ? u.z : u.w;
    return (j & 1) ? (w >> 16) : (w & 0xffffu);
  }

  __device__ __forceinline__ static uint32_t word32(const uint4& u, int j) {
    return j == 0 ? u.x : j == 1 ? u.y : j == 2 ? u.z : u.w;
  }

  // transposed: thread holds k-rows kb*4..kb*4+3 of columns mb*VEC..+VEC;
  // writes VEC LDS rows, each with 4 consecutive k values.
  __device__ __forceinline__ static void store_trans(char* lds, const uint4 (&v)[4]) {
    const int tid = threadIdx.x;
    const int mb = tid % MBC, kb = tid / MBC;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint2 w;
        w.x = half16(v[0], j) | (half16(v[1], j) << 16);
        w.y = half16(v[2], j) | (half16(v[3], j) << 16);
        *reinterpret_cast<uint2*>(lds + (mb * 8 + j) * ROW + kb * 8) = w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint4 w = make_uint4(word32(v[0], j), word32(v[1], j), word32(v[2], j), word32(v[3], j));
        *reinterpret_cast<uint4*>(lds + (mb * 4 + j) * ROW + kb * 16) = w;
      }
    }
  }
};

template <typename T>
__device__ __forceinline__ void mma_stage(const char* As, const char* Bs, f32x16_t (&acc)[2][2]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
  for (int chunk = 0; chunk < KBYTES / 32; ++chunk) {
    uint4 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      a[i] = *reinterpret_cast<const uint4*>(As + (wm * 64 + i * 32 + r32) * ROW + chunk * 32 + half * 16);
      b[i] = *reinterpret_cast<const uint4*>(Bs + (wn * 64 + i * 32 + r32) * ROW + chunk * 32 + half * 16);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (sizeof(T) == 2) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[i]),
                                                             __builtin_bit_cast(bf16x8_t, b[j]),
                                                             acc[i][j], 0, 0, 0);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[i].x), __uint_as_float(b[j].x),
                                                          acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[i].y), __uint_as_float(b[j].y),
                                                          acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[i].z), __uint_as_float(b[j].z),
                                                          acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[i].w), __uint_as_float(b[j].w),
                                                          acc[i][j], 0, 0, 0);
        }
      }
    }
  }
}

// Computes one tile and hands every accumulator to epi(row, col, value) with
// row, col the coordinates inside the 128x128 tile.  Each lane owns 4
// consecutive rows of one column per 32x32 block.  K is the contraction length.
template <typename T, bool TRANS_A, bool TRANS_B, class Epi>
__device__ __forceinline__ void tile(char* lds, const Operand& A, const Operand& B, int K, Epi&& epi) {
  using L = Loader<T>;
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  L la, lb;
  if constexpr (!TRANS_A) la.init_direct(A);
  if constexpr (!TRANS_B) lb.init_direct(B);
  const int nk = (K + L::BKE - 1) / L::BKE;
  __syncthreads();  // the previous user of this LDS is done
  if (nk > 0) {
    uint4 ra[4], rb[4];
    if constexpr (TRANS_A) L::load_trans(A, 0, ra); else la.load_direct(A, 0, ra);
    if constexpr (TRANS_B) L::load_trans(B, 0, rb); else lb.load_direct(B, 0, rb);
    if constexpr (TRANS_A) L::store_trans(lds, ra); else L::store_direct(lds, ra);
    if constexpr (TRANS_B) L::store_trans(lds + A_BYTES, rb); else L::store_direct(lds + A_BYTES, rb);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      char* cur = lds + (kt & 1) * STAGE;
      char* nxt = lds + ((kt + 1) & 1) * STAGE;
      const bool more = kt + 1 < nk;
      if (more) {
        if constexpr (TRANS_A) L::load_trans(A, kt + 1, ra); else la.load_direct(A, kt + 1, ra);
        if constexpr (TRANS_B) L::load_trans(B, kt + 1, rb); else lb.load_direct(B, kt + 1, rb);
      }
      mma_stage<T>(cur, cur + A_BYTES, acc);
      if (more) {
        if constexpr (TRANS_A) L::store_trans(nxt, ra); else L::store_direct(nxt, ra);
        if constexpr (TRANS_B) L::store_trans(nxt + A_BYTES, rb); else L::store_direct(nxt + A_BYTES, rb);
      }
      __syncthreads();
    }
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w & 1, wn = w >> 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int col = wn * 64 + j * 32 + (lane & 31);
        epi(row, col, acc[i][j][r]);
      }
}

}  // namespace gemm
}  // namespace moe
