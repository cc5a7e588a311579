// ragged_mm on CDNA4 matrix cores: one 128x128 output tile of a grouped
// (per-expert) matrix product, computed by one 256-thread workgroup.
//
// The Latch pages ("What Latch does", steps 1 and 3) name ragged_mm as the
// grouped expert product whose bucket sizes change every update, with
// derivative rules for its backward.  Here each tile is C[m,n] = sum_k A[m,k]
// B[k,n] with fp32 accumulation on MFMA (bf16: v_mfma_f32_32x32x16_bf16; fp32
// mode: v_mfma_f32_32x32x2_f32), four wavefronts of 64x64 each.
//
// Each operand is read from global memory in whichever orientation it is
// stored, always 16 contiguous bytes per lane, and copied to LDS unchanged:
//  * K-rows operand ("k runs along the source row": activations in the forward
//    products, weights read as W^T): LDS [m or n][k], 128 bytes of k per row;
//    an MFMA fragment is one ds_read_b128.
//  * MN-rows operand ("m or n runs along the source row": weights read as W,
//    and both operands of the weight-gradient products, where k runs over the
//    routed tokens): LDS [k][m or n], 256 bytes per row; in bf16 an MFMA
//    fragment is two ds_read_b64_tr_b16, the gfx950 LDS read that transposes
//    16-bit data across each group of 16 lanes.  (fp32 mode has no such read;
//    its MN-rows operands are transposed in registers before the LDS write.)
// Row indices may go through a map (the dispatch gather on load: row =
// perm[p] / k, used by the fp32 path; the bf16 path reads a gathered copy).
// bf16 tiles stage k-tiles through NS LDS buffers with direct-to-LDS loads
// (NS - 1 k-tiles in flight while the matrix cores work on one); fp32 tiles
// use two register-staged buffers.
#pragma once

#include "device_common.h"

namespace moe {
namespace gemm {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int KBYTES = 128;              // bytes of k per stage
constexpr int ROW = KBYTES + 16;         // LDS row stride of a K-rows operand (bytes)
constexpr int ROWT = 2 * KBYTES + 32;    // LDS row stride of an MN-rows bf16 operand (bytes)
constexpr int OP_BYTES = BM * ROW;       // one operand, one stage (both layouts fit)
constexpr int A_BYTES = OP_BYTES;
constexpr int STAGE = 2 * OP_BYTES;
constexpr int LDS_BYTES = 2 * STAGE;     // 73,728 bytes
static_assert((KBYTES / 2) * ROWT <= OP_BYTES, "MN-rows stage must fit");

// One operand of a tile.
//   K-rows:  logical row r (0..127) -> source row map(p0 + r), k runs along it;
//            rows r >= nrows and k >= lim read as zero.
//   MN-rows: logical k-row kk -> source row map(p0 + kk), the tile's m/n columns
//            mn0.. run along it; k-rows kk >= nrows and columns >= lim read as zero.
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

constexpr int CROW = BN + 4;   // fp32 words per LDS row of the staged tile
static_assert(BM * CROW * 4 <= LDS_BYTES, "staged tile must fit");

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;

template <typename T, bool MN>
struct Stager {
  static constexpr int VEC = 16 / (int)sizeof(T);      // elements per 16 bytes
  static constexpr int BKE = KBYTES / (int)sizeof(T);  // k elements per stage
  static constexpr bool TR_READ = MN && sizeof(T) == 2;  // LDS [k][mn], transpose on read

  // source byte offsets of this thread's 4 rows (-1 = out of range); only
  // K-rows operands keep them (their rows do not change along k)
  long rowoff[4];

  __device__ __forceinline__ void init(const Operand& o) {
    if constexpr (!MN) {
      const int tid = threadIdx.x;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = (tid >> 3) + 32 * i;
        rowoff[i] = (r < o.nrows) ? map_row(o, o.p0 + r) * o.ld * (long)sizeof(T) : -1;
      }
    }
  }

  // Out-of-range elements are loaded from the operand's first element (always
  // valid when a tile exists) and then zeroed, so every load is issued.
  __device__ __forceinline__ void load(const Operand& o, int kt, uint4 (&v)[4]) const {
    const int tid = threadIdx.x;
    if constexpr (!MN) {
      const int col = kt * BKE + (tid & 7) * VEC;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = rowoff[i] >= 0 && col < o.lim;
        uint4 x = *reinterpret_cast<const uint4*>(o.base + (ok ? rowoff[i] + (long)col * (long)sizeof(T) : 0L));
        if (!ok) x = make_uint4(0u, 0u, 0u, 0u);
        v[i] = x;
      }
    } else if constexpr (TR_READ) {
      // 64 k-rows x 256 bytes: 16 lanes per row, 16 rows per pass
      const int mn = o.mn0 + (tid & 15) * VEC;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = kt * BKE + (tid >> 4) + 16 * i;
        const bool ok = kk < o.nrows && mn < o.lim;
        const long off = ok ? (map_row(o, o.p0 + kk) * o.ld + mn) * (long)sizeof(T) : 0L;
        uint4 x = *reinterpret_cast<const uint4*>(o.base + off);
        if (!ok) x = make_uint4(0u, 0u, 0u, 0u);
        v[i] = x;
      }
    } else {
      // fp32: a block of 4 k-rows x 4 columns per thread
      const int mb = tid & 31, kb = tid >> 5;
      const int mn = o.mn0 + mb * VEC;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = kt * BKE + kb * 4 + i;
        const bool ok = kk < o.nrows && mn < o.lim;
        const long off = ok ? (map_row(o, o.p0 + kk) * o.ld + mn) * (long)sizeof(T) : 0L;
        uint4 x = *reinterpret_cast<const uint4*>(o.base + off);
        if (!ok) x = make_uint4(0u, 0u, 0u, 0u);
        v[i] = x;
      }
    }
  }

  __device__ __forceinline__ static uint32_t word32(const uint4& u, int j) {
    return j == 0 ? u.x : j == 1 ? u.y : j == 2 ? u.z : u.w;
  }

  __device__ __forceinline__ static void store(char* lds, const uint4 (&v)[4]) {
    const int tid = threadIdx.x;
    if constexpr (!MN) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(lds + ((tid >> 3) + 32 * i) * ROW + (tid & 7) * 16) = v[i];
    } else if constexpr (TR_READ) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(lds + ((tid >> 4) + 16 * i) * ROWT + (tid & 15) * 16) = v[i];
    } else {
      const int mb = tid & 31, kb = tid >> 5;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 w = make_uint4(word32(v[0], j), word32(v[1], j), word32(v[2], j), word32(v[3], j));
        *reinterpret_cast<uint4*>(lds + (mb * 4 + j) * ROW + kb * 16) = w;
      }
    }
  }

  // The 16-byte MFMA fragment of 32-row block `row0` (m or n), k chunk `chunk`
  // (32 bytes of k) for this lane: row row0 + lane%32, k elements
  // chunk*32/sizeof(T) + (lane/32)*VEC .. +VEC.
  __device__ __forceinline__ static uint4 frag(const char* lds, int row0, int chunk) {
    const int lane = threadIdx.x & 63;
    if constexpr (TR_READ) {
      // lane j of each 16-lane group points at k-row k0 + j/4, columns
      // c0 + 4*(j%4)..+3; lane i then holds k-rows k0..k0+3 of column c0 + i
      const int g = lane >> 4, j = lane & 15;
      const int k0 = chunk * 16 + 8 * (g >> 1);
      const int c0 = row0 + 16 * (g & 1);
      const char* p = lds + (k0 + (j >> 2)) * ROWT + (c0 + 4 * (j & 3)) * 2;
      const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)p);
      const v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(p + 4 * ROWT));
      uint4 r;
      r.x = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
      r.y = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
      r.z = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
      r.w = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
      return r;
    } else {
      return *reinterpret_cast<const uint4*>(lds + (row0 + (lane & 31)) * ROW + chunk * 32 + (lane >> 5) * 16);
    }
  }
};

// GELU applied to the 16 bytes of an A fragment as they come out of LDS (the
// recomputation rule: the stored tensor is H and the product needs gelu(H)):
// 8 bf16 values rounded back to bf16, or 4 fp32 values.
template <typename T>
__device__ __forceinline__ void gelu_frag(uint4& v) {
  uint32_t* w = &v.x;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if constexpr (sizeof(T) == 2)
      w[q] = pack_bf16x2(gelu_only(bf16_to_f32(w[q] & 0xffffu)), gelu_only(bf16_to_f32(w[q] >> 16)));
    else
      w[q] = __float_as_uint(gelu_only(__uint_as_float(w[q])));
  }
}

template <typename T, bool MN_A, bool MN_B, bool GA>
__device__ __forceinline__ void mma_stage(const char* As, const char* Bs, f32x16_t (&acc)[2][2]) {
  using SA = Stager<T, MN_A>;
  using SB = Stager<T, MN_B>;
  const int w = threadIdx.x >> 6;
  const int wm = w & 1, wn = w >> 1;
#pragma unroll
  for (int chunk = 0; chunk < KBYTES / 32; ++chunk) {
    uint4 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      a[i] = SA::frag(As, wm * 64 + i * 32, chunk);
      b[i] = SB::frag(Bs, wn * 64 + i * 32, chunk);
      if constexpr (GA) gelu_frag<T>(a[i]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (sizeof(T) == 2) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, b[j]),
                                                             __builtin_bit_cast(bf16x8_t, a[i]),
                                                             acc[i][j], 0, 0, 0);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(b[j].x), __uint_as_float(a[i].x),
                                                          acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(b[j].y), __uint_as_float(a[i].y),
                                                          acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(b[j].z), __uint_as_float(a[i].z),
                                                          acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(b[j].w), __uint_as_float(a[i].w),
                                                          acc[i][j], 0, 0, 0);
        }
      }
    }
  }
}

// Computes one tile, then hands it to the epilogue in row-major pieces: the
// accumulators go through LDS (fp32, 128 x 132) and epi(row, col, v) is called
// with 8 consecutive columns v[0..7] of one row (col a multiple of 8), so the
// epilogue's global accesses are 16- or 32-byte vectors and its code exists
// once instead of once per accumulator.  K is the contraction length; MN_A /
// MN_B select the MN-rows layout for that operand.

// No per-piece inputs for the epilogue.
struct NoPre {
  __device__ __forceinline__ int operator()(int, int) const { return 0; }
};

// Stages the accumulators through LDS (fp32, 128 x CROW) and calls epi(row,
// col, v) on 8-column row pieces.  The caller has made the LDS free.  With a
// `pre` functor, pre(row, col) is called for all of this thread's pieces
// first, so the global loads it makes (inputs of the epilogue) are all in
// flight together, and epi(row, col, v, pre_value) gets its result.
template <class Epi, class Pre>
__device__ __forceinline__ void epilogue(char* lds, const f32x16_t (&acc)[2][2], Epi&& epi, Pre&& pre) {
  constexpr int kIt = BM * (BN / 8) / kThreads;
  constexpr bool kPre = !__is_same(__remove_cvref(Pre), NoPre);
  using PV = decltype(pre(0, 0));
  PV pv[kPre ? kIt : 1];
  if constexpr (kPre) {
#pragma unroll
    for (int j = 0; j < kIt; ++j) {
      const int it = threadIdx.x + j * kThreads;
      pv[j] = pre(it >> 4, (it & 15) * 8);
    }
  }
  float* cs = reinterpret_cast<float*>(lds);
  {
    // every product is issued with its operands exchanged (B fragment first),
    // so accumulator block (i, j) holds its block transposed: lane l, register
    // r holds tile row 64 wm + 32 i + l % 32, column 64 wn + 32 j + 8 (r / 4) +
    // 4 (l / 32) + r % 4 -- four consecutive columns per register group, one
    // 16-byte LDS write each (rows CROW * 4 = 528 bytes apart, so 16
    // consecutive lanes cover all 64 banks)
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w & 1, wn = w >> 1;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row = wm * 64 + i * 32 + (lane & 31);
          const int col = wn * 64 + j * 32 + g * 8 + (lane >> 5) * 4;
          *reinterpret_cast<float4*>(cs + row * CROW + col) =
              make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
        }
  }
  lds_sync();
  if constexpr (kPre) {
#pragma unroll
    for (int j = 0; j < kIt; ++j) {
      const int it = threadIdx.x + j * kThreads;
      const int row = it >> 4, col = (it & 15) * 8;
      const float4 lo = *reinterpret_cast<const float4*>(cs + row * CROW + col);
      const float4 hi = *reinterpret_cast<const float4*>(cs + row * CROW + col + 4);
      float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      epi(row, col, v, pv[j]);
    }
  } else {
#pragma unroll 1
    for (int it = threadIdx.x; it < BM * (BN / 8); it += kThreads) {
      const int row = it >> 4, col = (it & 15) * 8;
      const float4 lo = *reinterpret_cast<const float4*>(cs + row * CROW + col);
      const float4 hi = *reinterpret_cast<const float4*>(cs + row * CROW + col + 4);
      float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      epi(row, col, v);
    }
  }
}

template <typename T, bool MN_A, bool MN_B, bool GA, class Epi, class Pre>
__device__ __forceinline__ void tile_reg(char* lds, const Operand& A, const Operand& B, int K, Epi&& epi, Pre&& pre) {
  using SA = Stager<T, MN_A>;
  using SB = Stager<T, MN_B>;
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  SA sa;
  SB sb;
  sa.init(A);
  sb.init(B);
  const int nk = (K + SA::BKE - 1) / SA::BKE;
  __syncthreads();  // the previous user of this LDS is done
  if (nk > 0) {
    uint4 ra[4], rb[4];
    sa.load(A, 0, ra);
    sb.load(B, 0, rb);
    SA::store(lds, ra);
    SB::store(lds + A_BYTES, rb);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      char* cur = lds + (kt & 1) * STAGE;
      char* nxt = lds + ((kt + 1) & 1) * STAGE;
      const bool more = kt + 1 < nk;
      if (more) {
        sa.load(A, kt + 1, ra);
        sb.load(B, kt + 1, rb);
      }
      mma_stage<T, MN_A, MN_B, GA>(cur, cur + A_BYTES, acc);
      if (more) {
        SA::store(nxt, ra);
        SB::store(nxt + A_BYTES, rb);
      }
      __syncthreads();
    }
  }
  epilogue(lds, acc, epi, pre);
}


// ---------------------------------------------------------------------------
// bf16 tiles: direct-to-LDS loads (buffer_load_dwordx4 ... lds), up to four
// LDS stages, so the loads of three k-tiles are in flight while the matrix
// cores work on the fourth, at no register cost.  Each wave instruction fills
// 1 KB of LDS contiguously (lane l -> bytes 16l..16l+15), so bank conflicts on
// the MFMA reads are avoided by an XOR swizzle of 16-byte units instead of
// padding:
//  * K-rows operand, LDS [128 rows][128 B]: logical k-unit u of row r sits in
//    physical unit u ^ ((r >> 1) & 7);
//  * MN-rows operand, LDS [64 k-rows][256 B]: logical 16-byte column slot s of
//    k-row r sits in physical slot s ^ (4 * (r & 3)).  Half a transpose read
//    (32 lanes) covers 4 k-rows x 64 bytes; the XOR puts the 4 rows' 64-byte
//    pieces in the 4 distinct quarters of the 64 banks.
// Out-of-range elements are zeroed by the loads' range check.  The loop waits
// on the vector-memory counter itself and synchronises with a bare s_barrier,
// so the loads of later k-tiles stay in flight across it.
// ---------------------------------------------------------------------------
constexpr int DMA_OP = 16384;                  // bytes per operand per stage
constexpr int DMA_STAGE = 2 * DMA_OP;
// LDS of a tile with NS stages: the stages, or the staged fp32 tile of the
// epilogue if that is larger (4 stages: 131,072 bytes; 2 stages: 67,584)
constexpr int dma_lds_bytes(int NS) { return NS * DMA_STAGE > BM * CROW * 4 ? NS * DMA_STAGE : BM * CROW * 4; }

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)p);
}

// s_waitcnt vmcnt(n) for n in {0, 8, 16}; expcnt and lgkmcnt left alone
__device__ __forceinline__ void wait_vm(int outstanding_tiles) {
  if (outstanding_tiles >= 2) __builtin_amdgcn_s_waitcnt(0x4F70);
  else if (outstanding_tiles == 1) __builtin_amdgcn_s_waitcnt(0x0F78);
  else __builtin_amdgcn_s_waitcnt(0x0F70);
}

__device__ __forceinline__ void lds_barrier() {
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

// The direct-to-LDS loads of one operand, as buffer loads.  Wave w's
// instruction i (0..3) fills LDS bytes [1024 (4w + i), +1024) of the
// operand's stage:
//  * K-rows: LDS row r = 8 (4w + i) + lane / 8 (128 bytes of k), physical
//    16-byte unit lane % 8, which holds logical k-unit u = (lane % 8) ^
//    ((4i + lane / 16) % 8) (the swizzle u ^ ((r / 2) % 8));
//  * MN-rows: k-row kk = 16w + 4i + lane / 16 of the stage, physical slot
//    lane % 16, which holds columns mn0 + 8 s.. with s = (lane % 16) ^
//    4 ((lane / 16) % 4) (the swizzle s ^ 4 (kk % 4)).
// Every load goes through one wave-uniform buffer descriptor per operand and
// k-tile whose base is the tile's source in that k-tile (a scalar 64-bit add
// per k-tile); each lane keeps a fixed 32-bit offset from it per instruction.
// Out-of-range elements come back as zeros from the descriptor's range check:
// a lane whose row (K-rows) or column (MN-rows) lies outside the operand gets
// offset kOutside, at or beyond any record count; for MN-rows the record
// count of k-tile kt is the bytes of rows still in range from its base, so
// the ragged k-rows of the last k-tile read as zero.  A K-rows operand whose
// k extent is not a multiple of 64 re-derives its offsets in the last k-tile.
// Issuing a k-tile so costs scalar work only (plus that one tail).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutside = 0x80000000u;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer: 32-bit data format, no swizzle

__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

template <bool MN>
struct DmaOp {
  uint64_t base;       // source of k-tile 0 (wave-uniform)
  uint64_t step;       // source bytes per k-tile (wave-uniform)
  int lim;             // K-rows: k elements in range; MN-rows: k-rows in range
  int rowbytes;        // MN-rows: bytes per k-row (ld * 2)
  int caprows;         // MN-rows: k-rows whose bytes stay below kOutside
  uint32_t voff[4];    // this lane's offset from the k-tile's base, per instruction
  uint32_t wofs;       // this wave's LDS byte offset within an operand stage (wave-uniform)

  __device__ __forceinline__ void init(const Operand& o) {
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    wofs = (uint32_t)w * 4096u;
    if constexpr (!MN) {
      base = uniform_u64((uint64_t)(uintptr_t)(o.base + (long)o.p0 * o.ld * 2));
      step = 128;
      lim = __builtin_amdgcn_readfirstlane(o.lim);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 8 * (4 * w + i) + (lane >> 3);
        const int unit = (lane & 7) ^ ((4 * i + (lane >> 4)) & 7);
        voff[i] = row < o.nrows ? (uint32_t)(row * o.ld * 2 + unit * 16) : kOutside;
      }
    } else {
      base = uniform_u64((uint64_t)(uintptr_t)(o.base + ((long)o.p0 * o.ld + o.mn0) * 2));
      step = uniform_u64((uint64_t)(128L * o.ld));
      lim = __builtin_amdgcn_readfirstlane(o.nrows);
      rowbytes = __builtin_amdgcn_readfirstlane((int)o.ld * 2);
      caprows = (int)(kOutside / (uint32_t)rowbytes);
      const int slot = (lane & 15) ^ (4 * ((lane >> 4) & 3));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk0 = 16 * w + 4 * i + (lane >> 4);
        voff[i] = o.mn0 + slot * 8 < o.lim ? (uint32_t)(kk0 * o.ld * 2 + slot * 16) : kOutside;
      }
    }
  }

  // the loads of k-tile kt into the operand stage at LDS byte address lst
  __device__ __forceinline__ void issue(int kt, uint32_t lst) const {
    const uint32_t lbase = lst + wofs;
    const uint64_t b = base + (uint64_t)kt * step;
    // K-rows: k elements of this k-tile in range; MN-rows: k-rows in range
    const int left = lim - 64 * kt;
    uint32_t nrec = kOutside;
    if constexpr (MN) nrec = left <= 0 ? 0u : left >= caprows ? kOutside : (uint32_t)(left * rowbytes);
    const rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)b, (short)0, (int)nrec, kRsrcWord3);
    if (MN || __builtin_expect(left >= 64, 1)) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(uintptr_t)(lbase + 1024u * i), 16, (int)voff[i],
                                                 0, 0, 0);
    } else {
      // the last k-tile of a K-rows operand whose k extent is not a multiple
      // of 64: units at or beyond the limit read as zero
      const int lane = threadIdx.x & 63;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int unit = (lane & 7) ^ ((4 * i + (lane >> 4)) & 7);
        const uint32_t v = unit * 8 < left ? voff[i] : kOutside;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(uintptr_t)(lbase + 1024u * i), 16, (int)v, 0, 0,
                                                 0);
      }
    }
  }
};

// LDS reads of data written by the direct-to-LDS loads are issued as inline
// assembly that ends in its own lgkmcnt wait: the compiler cannot tell that
// they read a different stage than the loads still in flight and would
// otherwise drain every outstanding load before each read.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

// Byte offset of this lane's fragment within an operand stage (K-rows: the
// b128 read; MN-rows: the first of the two transpose reads, the second is
// 1024 bytes further).
template <bool MN>
__device__ __forceinline__ uint32_t dma_frag_off(int row0, int chunk) {
  const int lane = threadIdx.x & 63;
  if constexpr (!MN) {
    const int r = row0 + (lane & 31);
    const int u = chunk * 2 + (lane >> 5);
    return (uint32_t)(r * 128 + ((u ^ ((r >> 1) & 7)) << 4));
  } else {
    const int g = lane >> 4, j = lane & 15;
    const int r = chunk * 16 + 8 * (g >> 1) + (j >> 2);
    const int c = row0 + 16 * (g & 1) + 4 * (j & 3);
    return (uint32_t)(r * 256 + (((c >> 3) ^ (4 * (r & 3))) << 4) + (c & 7) * 2);
  }
}

// LDS addresses of one operand's fragments for this lane, split into a
// register and an instruction offset.  Within a stage, the two 32-row blocks
// of a K-rows operand are 4096 bytes apart (rows r and r + 32 share the
// swizzle), so a register per k chunk serves both; the k chunks of an MN-rows
// operand are 4096 bytes apart (16 k-rows), so a register per row block
// serves all four.  The stage slot's offset is added to the register.
template <bool MN>
struct FragAddr {
  static constexpr int NREG = MN ? 2 : 4;
  uint32_t r[NREG];

  __device__ __forceinline__ void init(uint32_t op0, int row0) {
#pragma unroll
    for (int q = 0; q < NREG; ++q)
      r[q] = op0 + (MN ? dma_frag_off<true>(row0 + 32 * q, 0) : dma_frag_off<false>(row0, q));
  }
  // row block I (0, 1), k chunk C (0..3)
  template <int I, int C>
  __device__ __forceinline__ uint32_t reg() const {
    return r[MN ? I : C];
  }
  template <int I, int C>
  static constexpr int imm() {
    return MN ? C * 4096 : I * 4096;
  }
};

// The fragments of one 16-element k chunk: a0/a1 for the two 32-row blocks of
// A (m), b0/b1 for those of B (n), 8 bf16 per lane each.
struct Frags {
  u32x4_t a0, a1, b0, b1;
};

// GELU on both A fragments of a chunk (bf16, the direct-to-LDS path).  It is
// called right after the pipeline block whose wait completes the fragments'
// LDS reads.  To the compiler those registers were written by an earlier asm
// statement, so it could hoist this arithmetic above the waiting block and read
// them before the data lands; the empty volatile asm with in/out operands
// stays after that block (volatile asm statements keep their order) and the
// arithmetic depends on its outputs.
__device__ __forceinline__ void gelu_a(Frags& f) {
  asm volatile("" : "+v"(f.a0), "+v"(f.a1));
  uint4 a0 = {f.a0[0], f.a0[1], f.a0[2], f.a0[3]}, a1 = {f.a1[0], f.a1[1], f.a1[2], f.a1[3]};
  gelu_frag<uint16_t>(a0);
  gelu_frag<uint16_t>(a1);
  f.a0 = u32x4_t{a0.x, a0.y, a0.z, a0.w};
  f.a1 = u32x4_t{a1.x, a1.y, a1.z, a1.w};
}

__device__ __forceinline__ u32x4_t join(const u32x2_t& lo, const u32x2_t& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
}

// The k loop is software-pipelined by hand, two chunks deep: one asm block
// issues the LDS reads of chunk c+2, runs the four MFMAs of chunk c, and then
// waits only for the reads of chunk c+1 (issued one block earlier), so every
// read has two blocks of matrix work to land.  Reads, MFMAs and the wait share
// one block, and the fragments of chunk c+2 are next touched two blocks later,
// after the wait that completes them; the compiler is never handed a register
// whose read it could observe early.  Accumulators live in AGPRs.
//   WAIT = 0: wait for every read; 1: leave this block's reads outstanding;
//   -1: no wait.
#define MOE_RD_K(d, a) "ds_read_b128 %[" d "], %[" a "] offset:%[o" a "]\n\t"
#define MOE_RD_MN(d, a) \
  "ds_read_b64_tr_b16 %[" d "l], %[" a "] offset:%[o" a "]\n\tds_read_b64_tr_b16 %[" d "h], %[" a "] offset:%[o" a "h]\n\t"
#define MOE_MFMA4                                                   \
  "v_mfma_f32_32x32x16_bf16 %[c00], %[b0], %[a0], %[c00]\n\t"      \
  "v_mfma_f32_32x32x16_bf16 %[c01], %[b1], %[a0], %[c01]\n\t"      \
  "v_mfma_f32_32x32x16_bf16 %[c10], %[b0], %[a1], %[c10]\n\t"      \
  "v_mfma_f32_32x32x16_bf16 %[c11], %[b1], %[a1], %[c11]\n\t"
#define MOE_ACC_OUT [c00] "+a"(acc[0][0]), [c01] "+a"(acc[0][1]), [c10] "+a"(acc[1][0]), [c11] "+a"(acc[1][1])
#define MOE_CUR_IN [a0] "v"(c.a0), [a1] "v"(c.a1), [b0] "v"(c.b0), [b1] "v"(c.b1)
#define MOE_ADDR_IN                                                                                  \
  [pa0] "v"(pa0), [pa1] "v"(pa1), [pb0] "v"(pb0), [pb1] "v"(pb1), [opa0] "i"(OA0), [opa0h] "i"(OA0 + 1024), \
      [opa1] "i"(OA1), [opa1h] "i"(OA1 + 1024), [opb0] "i"(OB0), [opb0h] "i"(OB0 + 1024), [opb1] "i"(OB1),  \
      [opb1h] "i"(OB1 + 1024)
// one pipeline block for a layout pair: READS issues the reads into the
// output operands OUTS; NREAD is the number of LDS instructions in READS
#define MOE_PIPE_BODY(READS, OUTS, NREAD, FINISH)                                                         \
  if constexpr (MMA && WAIT == 0) {                                                                      \
    asm volatile(READS MOE_MFMA4 "s_waitcnt lgkmcnt(0)" : OUTS, MOE_ACC_OUT : MOE_CUR_IN, MOE_ADDR_IN : "memory"); \
  } else if constexpr (MMA && WAIT == 1) {                                                               \
    asm volatile(READS MOE_MFMA4 "s_waitcnt lgkmcnt(" #NREAD ")"                                          \
                 : OUTS, MOE_ACC_OUT : MOE_CUR_IN, MOE_ADDR_IN : "memory");                              \
  } else if constexpr (MMA) {                                                                            \
    asm volatile(READS MOE_MFMA4 : OUTS, MOE_ACC_OUT : MOE_CUR_IN, MOE_ADDR_IN : "memory");              \
  } else if constexpr (WAIT == 0) {                                                                      \
    asm volatile(READS "s_waitcnt lgkmcnt(0)" : OUTS : MOE_ADDR_IN : "memory");                           \
  } else {                                                                                               \
    asm volatile(READS : OUTS : MOE_ADDR_IN : "memory");                                                 \
  }                                                                                                      \
  FINISH

#define MOE_PIPE_OUTS_KM [x0] "=&v"(x0), [x1] "=&v"(x1), [y0l] "=&v"(y0l), [y0h] "=&v"(y0h), [y1l] "=&v"(y1l), [y1h] "=&v"(y1h)
#define MOE_PIPE_OUTS_KK [x0] "=&v"(x0), [x1] "=&v"(x1), [y0] "=&v"(y0), [y1] "=&v"(y1)
#define MOE_PIPE_OUTS_MM [x0l] "=&v"(x0l), [x0h] "=&v"(x0h), [x1l] "=&v"(x1l), [x1h] "=&v"(x1h), [y0l] "=&v"(y0l), [y0h] "=&v"(y0h), [y1l] "=&v"(y1l), [y1h] "=&v"(y1h)

template <bool MN_A, bool MN_B>
struct Pipe;

// A K-rows, B MN-rows (forward products)
template <>
struct Pipe<false, true> {
  template <bool MMA, int WAIT, int OA0, int OA1, int OB0, int OB1>
  __device__ __forceinline__ static void step(Frags& n, const Frags& c, f32x16_t (&acc)[2][2], uint32_t pa0,
                                              uint32_t pa1, uint32_t pb0, uint32_t pb1) {
    u32x4_t x0, x1;
    u32x2_t y0l, y0h, y1l, y1h;
    MOE_PIPE_BODY(MOE_RD_K("x0", "pa0") MOE_RD_K("x1", "pa1") MOE_RD_MN("y0", "pb0") MOE_RD_MN("y1", "pb1"),
                  MOE_PIPE_OUTS_KM, 6,
                  n.a0 = x0; n.a1 = x1; n.b0 = join(y0l, y0h); n.b1 = join(y1l, y1h);)
  }
};

// both K-rows (dH = dO W2^T, dXs = dA W1^T)
template <>
struct Pipe<false, false> {
  template <bool MMA, int WAIT, int OA0, int OA1, int OB0, int OB1>
  __device__ __forceinline__ static void step(Frags& n, const Frags& c, f32x16_t (&acc)[2][2], uint32_t pa0,
                                              uint32_t pa1, uint32_t pb0, uint32_t pb1) {
    u32x4_t x0, x1, y0, y1;
    MOE_PIPE_BODY(MOE_RD_K("x0", "pa0") MOE_RD_K("x1", "pa1") MOE_RD_K("y0", "pb0") MOE_RD_K("y1", "pb1"),
                  MOE_PIPE_OUTS_KK, 4,
                  n.a0 = x0; n.a1 = x1; n.b0 = y0; n.b1 = y1;)
  }
};

// both MN-rows (weight gradients: k runs over the routed tokens)
template <>
struct Pipe<true, true> {
  template <bool MMA, int WAIT, int OA0, int OA1, int OB0, int OB1>
  __device__ __forceinline__ static void step(Frags& n, const Frags& c, f32x16_t (&acc)[2][2], uint32_t pa0,
                                              uint32_t pa1, uint32_t pb0, uint32_t pb1) {
    u32x2_t x0l, x0h, x1l, x1h, y0l, y0h, y1l, y1h;
    MOE_PIPE_BODY(MOE_RD_MN("x0", "pa0") MOE_RD_MN("x1", "pa1") MOE_RD_MN("y0", "pb0") MOE_RD_MN("y1", "pb1"),
                  MOE_PIPE_OUTS_MM, 8,
                  n.a0 = join(x0l, x0h); n.a1 = join(x1l, x1h); n.b0 = join(y0l, y0h); n.b1 = join(y1l, y1h);)
  }
};

// MFMAs of one chunk, no reads
template <bool MN_A, bool MN_B>
__device__ __forceinline__ void pipe_mma(const Frags& c, f32x16_t (&acc)[2][2]) {
  asm volatile(MOE_MFMA4 : MOE_ACC_OUT : MOE_CUR_IN);
}

#undef MOE_RD_K
#undef MOE_RD_MN
#undef MOE_MFMA4
#undef MOE_ACC_OUT
#undef MOE_CUR_IN
#undef MOE_ADDR_IN
#undef MOE_PIPE_BODY
#undef MOE_PIPE_OUTS_KM
#undef MOE_PIPE_OUTS_KK
#undef MOE_PIPE_OUTS_MM

// bf16 tile through the DMA pipeline.
//
// Schedule of k-tile kt (NS stages, slot kt % NS; the fragments of chunks 0
// and 1 are already read, F[c] holds chunk c):
//   MFMAs of chunk 0 | reads of chunk 2 -> F2 | wait for F1
//   MFMAs of chunk 1 | reads of chunk 3 -> F3 | wait for all: stage kt is in registers
//   wait for the loads of stage kt+1, barrier, issue the loads of stage
//   kt+NS into slot kt % NS (every wave is past its reads of it)
//   MFMAs of chunk 2 | reads of chunk 0 of stage kt+1 -> F0
//   MFMAs of chunk 3 | reads of chunk 1 of stage kt+1 -> F1 | wait for F0
// so NS - 1 k-tiles of loads are in flight while one is computed, and each
// LDS read has at least one block of matrix work to hide behind.  NS = 4 with
// one workgroup per compute unit; NS = 2 when two workgroups share one (each
// then has half the LDS, and the other workgroup's work covers the waits).

// one pipeline block reading chunk C of the stage at LDS offset so from the
// stage of slot 0
template <bool MMA, int WAIT, int C, bool MN_A, bool MN_B>
__device__ __forceinline__ void pipe_step(Frags& n, const Frags& c, f32x16_t (&acc)[2][2], const FragAddr<MN_A>& fa,
                                          const FragAddr<MN_B>& fb, uint32_t so) {
  using FA = FragAddr<MN_A>;
  using FB = FragAddr<MN_B>;
  Pipe<MN_A, MN_B>::template step<MMA, WAIT, FA::template imm<0, C>(), FA::template imm<1, C>(),
                                  FB::template imm<0, C>(), FB::template imm<1, C>()>(
      n, c, acc, fa.template reg<0, C>() + so, fa.template reg<1, C>() + so, fb.template reg<0, C>() + so,
      fb.template reg<1, C>() + so);
}

__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[2][2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// The k-loop of one tile over operands A, B (contraction length K), added
// into acc; no epilogue.  On return every load of the tile has completed.
template <int NS, bool MN_A, bool MN_B, bool GA>
__device__ __forceinline__ void tile_dma_acc(char* lds, const Operand& A, const Operand& B, int K,
                                             f32x16_t (&acc)[2][2]) {
  static_assert(NS >= 2 && NS <= 4, "wait_vm covers up to two k-tiles in flight behind the one awaited");
  DmaOp<MN_A> da;
  DmaOp<MN_B> db;
  da.init(A);
  db.init(B);
  const int nk = (K + 63) / 64;
  const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
  lds_sync();  // the previous user of this LDS is done (its global stores may still be in flight)
  for (int j = 0; j < NS - 1 && j < nk; ++j) {
    da.issue(j, l0 + j * DMA_STAGE);
    db.issue(j, l0 + j * DMA_STAGE + DMA_OP);
  }
  if (nk > 0) {
    const int w = threadIdx.x >> 6;
    const int wm = w & 1, wn = w >> 1;
    FragAddr<MN_A> fa;
    FragAddr<MN_B> fb;
    fa.init(l0, wm * 64);
    fb.init(l0 + DMA_OP, wn * 64);
    wait_vm(min(NS - 2, nk - 1));
    lds_barrier();
    if (NS - 1 < nk) {
      da.issue(NS - 1, l0 + (NS - 1) * DMA_STAGE);
      db.issue(NS - 1, l0 + (NS - 1) * DMA_STAGE + DMA_OP);
    }
    Frags F0, F1, F2, F3;
    // With GA, the A fragments of each chunk pass through GELU once their
    // reads have completed (after the wait that covers them) and before the
    // MFMAs that use them.
    pipe_step<false, -1, 0>(F0, F0, acc, fa, fb, 0u);
    pipe_step<false, 0, 1>(F1, F1, acc, fa, fb, 0u);
    if constexpr (GA) gelu_a(F0);
    for (int kt = 0; kt < nk - 1; ++kt) {
      const uint32_t so = (uint32_t)(kt % NS) * DMA_STAGE;
      const uint32_t sn = (uint32_t)((kt + 1) % NS) * DMA_STAGE;
      pipe_step<true, 1, 2>(F2, F0, acc, fa, fb, so);
      if constexpr (GA) gelu_a(F1);
      pipe_step<true, 0, 3>(F3, F1, acc, fa, fb, so);
      if constexpr (GA) {
        gelu_a(F2);
        gelu_a(F3);
      }
      // every stage up to min(kt + NS - 1, nk - 1) has all its loads issued
      wait_vm(min(NS - 2, nk - 2 - kt));
      lds_barrier();
      if (kt + NS < nk) {
        da.issue(kt + NS, l0 + so);
        db.issue(kt + NS, l0 + so + DMA_OP);
      }
      pipe_step<true, -1, 0>(F0, F2, acc, fa, fb, sn);
      pipe_step<true, 1, 1>(F1, F3, acc, fa, fb, sn);
      if constexpr (GA) gelu_a(F0);
    }
    {
      // last k-tile: its chunks 0 and 1 are in flight or landed
      const uint32_t so = (uint32_t)((nk - 1) % NS) * DMA_STAGE;
      pipe_step<true, 1, 2>(F2, F0, acc, fa, fb, so);
      if constexpr (GA) gelu_a(F1);
      pipe_step<true, 0, 3>(F3, F1, acc, fa, fb, so);
      if constexpr (GA) {
        gelu_a(F2);
        gelu_a(F3);
      }
      pipe_mma<MN_A, MN_B>(F2, acc);
      pipe_mma<MN_A, MN_B>(F3, acc);
    }
    // the MFMA results are read by ordinary code below: cover the
    // write-to-read distance the hardware requires after the last MFMA
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[1][0]), "+a"(acc[1][1]));
  }
}

template <int NS, bool MN_A, bool MN_B, bool GA, class Epi, class Pre>
__device__ __forceinline__ void tile_dma(char* lds, const Operand& A, const Operand& B, int K, Epi&& epi,
                                         Pre&& pre) {
  f32x16_t acc[2][2];
  zero_acc(acc);
  tile_dma_acc<NS, MN_A, MN_B, GA>(lds, A, B, K, acc);
  // every wave is done with the stages (all direct-to-LDS loads completed at
  // the last vmcnt wait, none was issued after it)
  lds_sync();
  epilogue(lds, acc, epi, pre);
}

// One bf16 tile whose contraction runs over n operand pieces: piece(i, A, B,
// K) fills the operands of piece i and returns false to skip it.  The pieces
// are added into one set of accumulators in order; one epilogue.
template <int NS, bool MN_A, bool MN_B, bool GA, class Piece, class Epi, class Pre>
__device__ __forceinline__ void tile_dma_pieces(char* lds, int n, Piece&& piece, Epi&& epi, Pre&& pre) {
  f32x16_t acc[2][2];
  zero_acc(acc);
  for (int i = 0; i < n; ++i) {
    Operand A, B;
    int K = 0;
    if (piece(i, A, B, K)) tile_dma_acc<NS, MN_A, MN_B, GA>(lds, A, B, K, acc);
  }
  lds_sync();
  epilogue(lds, acc, epi, pre);
}

// One tile: bf16 through the DMA pipeline (NS stages), fp32 through register
// staging.
// GA: the A operand holds H and the product uses gelu(H) (recomputation rule).
template <typename T, int NS, bool MN_A, bool MN_B, bool GA = false, class Epi, class Pre = NoPre>
__device__ __forceinline__ void tile(char* lds, const Operand& A, const Operand& B, int K, Epi&& epi,
                                     Pre&& pre = Pre()) {
  if constexpr (sizeof(T) == 2) tile_dma<NS, MN_A, MN_B, GA>(lds, A, B, K, epi, pre);
  else tile_reg<T, MN_A, MN_B, GA>(lds, A, B, K, epi, pre);
}

}  // namespace gemm
}  // namespace moe
