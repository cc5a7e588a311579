// The phases of one MoE-layer training update, as device functions of the
// persistent kernel.  Each phase is spread over every workgroup; phases that
// read results produced on other compute units are separated by a grid barrier
// (Latch pages, "What Latch does", step 4: work is grouped into phases that span
// every SM, a phase waits at a grid-wide barrier for data made on other SMs, and
// values that outlive a phase sit in a planned arena in GPU memory).
//
//   P0  bf16 weight copy refresh (optional); copy of W_r^T;
//       router logits, token_topk, gates, per-workgroup expert histogram
//   P1  route_order: global offsets, stable scatter into perm / inv; the
//       dispatch gather of the token rows into expert order (bf16)
//   P2  ragged_mm 1 + GELU        A = gelu(X_e W1[e]),  G' = gelu'(X_e W1[e])
//   P3  ragged_mm 2               O = A_e W2[e]
//   P4  weighted combine, loss, dL/dO, dL/dgate, dL/dlogit
//   P5  dH = (dO W2[e]^T) * G';  dW2[e] = A_e^T dO;  router-gradient partials
//   P6  dW1[e] = X_e^T dH;  dXs = dH W1[e]^T;  router gradient (fixed-order sum)
//   P7  dx = router part + the k expert contributions of each token, in order;
//       global norm from the per-tile partials (fixed order); clip + AdamW
#pragma once

#include "device_common.h"
#include "ragged_gemm.h"

namespace moe {

constexpr int kPhases = 8;
constexpr int kMetaBytes = 4096;
// microbatch slots of deferred expert weight gradients (one per launch of an
// update, from its first launch to the one that applies the experts)
constexpr int kMaxSlots = 16;
// OCC workgroups per compute unit: the kernel is built for one (all of a
// SIMD's registers per wave, 4-stage GEMM pipeline) or two (at most 256
// registers per wave, 2-stage pipeline, half the LDS each).
constexpr int dma_stages(int occ) { return occ == 1 ? 4 : 2; }
constexpr int scratch_bytes(int occ) {
  return gemm::LDS_BYTES > gemm::dma_lds_bytes(dma_stages(occ)) ? gemm::LDS_BYTES : gemm::dma_lds_bytes(dma_stages(occ));
}
constexpr int smem_bytes(int occ) { return kMetaBytes + scratch_bytes(occ); }
static_assert(2 * smem_bytes(2) <= 160 * 1024, "two workgroups per compute unit must fit the LDS");
// Tokens per router-gradient partial (a chunk of T x a 256-column block is one
// work item of the dH + dW2 phase): 128, halved down to 32 while the items
// are fewer than the workgroups, so a small batch spreads them over more
// workgroups in cheaper pieces.  The same rule sizes the partial buffer.
__host__ __device__ constexpr int router_chunk_tokens(int T, int d, int G) {
  const int cch = (d + kThreads - 1) / kThreads;
  int r = 128;
  while (r > 32 && ((T + r - 1) / r) * cch < G) r >>= 1;
  return r;
}

// Routing metadata kept in LDS for the whole launch (every workgroup computes
// it in P1 from the global histogram).
struct Meta {
  int cnt[kMaxExperts];         // routed rows per expert
  int off[kMaxExperts + 1];     // first sorted position of each expert
  int moff[kMaxExperts + 1];    // first 128-row tile of each expert
  int ord[kMaxExperts];         // experts by descending row count (ties: lower index first)
  int skewed;                   // some expert holds more than twice the mean rows
  // skewed routing: an expert's weight-gradient contraction is split into
  // chunks of kc rows (a multiple of 64, about twice the mean rows per expert)
  int kc;
  int nch[kMaxExperts];         // chunks of each expert (1 unless skewed)
  int pbase[kMaxExperts];       // first partial-tile block of each expert (sum of nch - 1 before it)
  int cpre[kMaxExperts + 1];    // chunks of the experts before rank r, in ord order
  int nsplit;                   // experts with more than one chunk
  int splitlist[kMaxExperts];   // those experts, ascending
  // skewed routing on a grid of 8 x P workgroups: the (expert, chunk) units of
  // the weight-gradient products, packed as expert | chunk << 8, longest
  // first; their tiles in that order (unit i holds tiles i*tpe .. i*tpe+tpe-1)
  // are split into 8 contiguous ranges of about equal cost, and [xb[h], xe[h])
  // is the range of this workgroup's XCD (x = b % 8) in the dW2 (h = 0) and
  // the dW1 (h = 1) phase, whose tiles weigh their fixed costs differently
  int nxu;
  int xb[2], xe[2];
  int xunit[3 * kMaxExperts + 1];   // E units plus the extra chunks (at most E under the rules below)
  float red[8];                 // block reductions
  BarrierState bar;             // grid-barrier bookkeeping (result broadcast, XCD membership)
  // rows of each expert that the weight-gradient products of this launch
  // contract over: its own (cnt), or with deferred weight gradients those of
  // every slot of the update in the applying launch and none in the others
  int wcnt[kMaxExperts];
  int wtot;
  // deferred weight gradients: one expert's rows (cnt, first sorted position)
  // in each slot, filled per tile
  int stab[2][kMaxSlots];
};
static_assert(sizeof(Meta) <= kMetaBytes, "meta");

struct KParams {
  // shape of this launch
  int T, d, f, E, k;
  float inv_tupd;     // 1 / tokens_in_update
  unsigned flags;
  // optimizer
  float lr, beta1, beta2, omb1, omb2, eps, wd, clip;
  float inv_bc1[2], inv_sqrt_bc2[2];   // AdamW bias corrections: [0] router, [1] experts
  unsigned epoch;     // launch number on this handle (barrier targets)
  int recompute;      // memory rule: act holds H (not gelu(H)) and there is no G' buffer
  // caller buffers
  const void* x;
  const void* t;
  const float* bias;
  float* params;
  float* grads;
  float* m;
  float* v;
  float* dx;
  float* stats;
  float* dbg_logits;
  int* dbg_idx;
  float* dbg_gate;
  int* dbg_counts;
  int* dbg_perm;
  uint64_t* trace;
  // arena
  int* idx;        // [T*k] expert of flat id i*k+j
  float* gate;     // [T*k]
  float* dzsel;    // [T*k] dL/dlogit of the selected experts
  int* hist;       // [G][E]
  int* ready;      // [nrb] GEMM-1 column tiles done per 128-row tile (readiness mode)
  int nrb;
  int* perm;       // [T*k] sorted position -> flat id
  int* inv;        // [T*k] flat id -> sorted position
  void* act;       // [N, f] gelu(H), or H under the recomputation rule   (T-typed)
  void* gp;        // [N, f] gelu'(H); unused under the recomputation rule (T-typed)
  float* out;      // [N, d] expert outputs O
  void* dout;      // [N, d] dL/dO              (T-typed)
  void* dh;        // [N, f] dL/dH              (T-typed)
  void* dxs;       // [T*k, d] per-(token, slot) input gradient (T-typed)
  float* wrt;      // [E, d] W_r^T as it was before this update
  float* rpart;    // [ceil(T/256)][E][d] router-gradient partials
  float* loss_part;  // [G]
  float* norm_part;  // [n10 + n11 + nr]
  uint16_t* shadow;  // [2*E*d*f] bf16 copy of W1 | W2 (bf16 mode)
  float* wpart2;     // partial dW2 tiles of split contractions [blocks][tiles per expert][128 x 128]
  float* wpart1;     // the same for dW1
  int wpart_sets;    // blocks each of them holds (extra chunks over all experts)
  int nt_stores;     // product outputs written with non-temporal stores (large launches)
  void* xs;          // [N, d] token rows in expert order (bf16 mode), written by route_order
  // deferred expert weight gradients (bf16): act, dout, xs and dh above are
  // this launch's slot of per-slot arrays; the launch that applies the
  // experts contracts dW1 / dW2 over the rows of slots 0..slot
  int defer;         // 1: weight gradients deferred to the applying launch
  int slot;          // this launch's slot
  int defer_final;   // this launch applies the experts: the dW products run, over every slot
  int defer_zero;    // the update's slot-0 launch zeroed the expert gradients (write, not add)
  const char* slot_act;   // slot 0 of act, dout, xs, dh; slot s at + s * stride
  const char* slot_dout;
  const char* slot_xs;
  const char* slot_dh;
  long stride_nf, stride_nd;   // bytes per slot of the [N, f] and [N, d] arrays
  int* slot_cnt;     // [kMaxSlots][E] rows of each expert per slot
  int* slot_off;     // [kMaxSlots][E] first sorted position of each expert per slot
  Ctrl ctrl;
};

__device__ __forceinline__ int logical_wg() {
  // Workgroups are dealt to the 8 XCDs round-robin; renumber so that
  // consecutive logical indices sit on the same XCD and share its L2.
  const int G = gridDim.x, b = blockIdx.x;
  if ((G & 7) != 0) return b;
  return (b & 7) * (G >> 3) + (b >> 3);
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Work items [0, n) of a phase, dealt so that each XCD gets one contiguous
// block of items (shared operands stay in that XCD's L2) and the blocks are
// equal to within one item.  Workgroup b runs on XCD b % 8.
struct Span {
  int begin, end, step;
  int begin2 = 0, end2 = 0, step2 = 1;   // an optional second run, taken after the first
  __device__ __forceinline__ int count() const {
    return max(0, ceil_div(end - begin, step)) + max(0, ceil_div(end2 - begin2, step2));
  }
  __device__ __forceinline__ int item(int i) const {
    const int c1 = max(0, ceil_div(end - begin, step));
    return i < c1 ? begin + i * step : begin2 + (i - c1) * step2;
  }
};
__device__ __forceinline__ Span xcd_span(int n) {
  const int G = gridDim.x;
  if ((G & 7) != 0) return {(int)blockIdx.x, n, G};
  const int x = blockIdx.x & 7, j = blockIdx.x >> 3, per = G >> 3;
  const int chunk = (n + 7) >> 3;
  const int lo = min(n, x * chunk);
  const int hi = min(n, lo + chunk);
  return {lo + j, hi, per};
}

// As xcd_span, but the XCD's items go to its workgroups from the last one
// down: a phase that deals several kinds of work gives its small trailing
// kind to the workgroups that got the fewest items of the kinds before it.
__device__ __forceinline__ Span xcd_span_last(int n) {
  const int G = gridDim.x;
  if ((G & 7) != 0) return {G - 1 - (int)blockIdx.x, n, G};
  const int x = blockIdx.x & 7, per = G >> 3, j = per - 1 - (int)(blockIdx.x >> 3);
  const int chunk = (n + 7) >> 3;
  const int lo = min(n, x * chunk);
  const int hi = min(n, lo + chunk);
  return {lo + j, hi, per};
}

// Weight-gradient tiles of all experts (tpe per expert).  Their contraction
// runs over the expert's rows, so under skewed routing the tiles of a heavy
// expert cost many times those of a light one.  Balanced routing keeps the
// XCD-contiguous deal of xcd_span (an expert's operands stay in one XCD's L2),
// one item per tile.  Skewed routing splits each expert's contraction into
// chunks of kc rows (item = expert, chunk, tile), takes the items in order of
// descending expert row count and deals them over all workgroups in a snake
// (0..G-1, G-1..0, ...), so every workgroup gets about the same sum of
// contraction lengths.
// Cost of a weight-gradient tile beyond its k-tiles, in k-tile units: the
// read-modify-write of its 64 KB fp32 gradient block and the epilogue.  Fitted
// to per-workgroup clocks under skewed Zipf routing (16 x 8192 tokens): in the
// dW2 phase about 9 us per tile against 0.4 us per k-tile of a long
// contraction, in the dW1 phase about 6 us against 0.55 us.
constexpr int kWTileFixed[2] = {24, 11};
static_assert(3 * kMaxExperts <= kThreads, "route_order ranks the weight-gradient units one per thread");
// route_order splits the tiles of both weight gradients (dW2: f x d, dW1: d x f)
// with one tile count per expert
static_assert(gemm::BM == gemm::BN, "square tiles: dW1 and dW2 have the same tiles per expert");
struct WItem {
  int e, c, t;   // expert, chunk, tile within the expert
};
// With a grid of 8 x P workgroups, skewed routing gives each XCD a contiguous
// range of the units' tiles (units longest first) of about equal cost, where a
// tile costs its k-tiles plus a fixed share for its fp32 gradient
// read-modify-write, which dominates a short contraction.  A unit's operand
// rows so go to one L2, or two where a range boundary splits it; the XCD's P
// workgroups take the range's tiles in a snake.
struct DealW {
  Span sp;
  bool snake, xl;
  int G, w, tpe, n, h;
  __device__ __forceinline__ int count() const {
    if (!snake) return sp.count();
    const int full = n / G, rem = n % G;   // rounds of G items, then a partial round
    const int last = (full & 1) ? G - 1 - w : w;
    return full + (last < rem ? 1 : 0);
  }
  // this workgroup's i-th item
  __device__ __forceinline__ WItem item(const Meta& meta, int E, int i) const {
    if (!snake) {
      const int q = sp.item(i);
      return {q / tpe, 0, q % tpe};
    }
    const int q = i * G + ((i & 1) ? G - 1 - w : w);
    if (xl) {
      const int g = meta.xb[h] + q;
      const int u = meta.xunit[g / tpe];
      return {u & 0xff, u >> 8, g % tpe};
    }
    int r = 0;
    while (r + 1 < E && meta.cpre[r + 1] * tpe <= q) ++r;
    const int rem = q - meta.cpre[r] * tpe;
    return {meta.ord[r], rem / tpe, rem % tpe};
  }
};
__device__ __forceinline__ DealW deal_weight_tiles(const Meta& meta, int E, int tpe, int h) {
  DealW dl;
  dl.h = h;
  dl.snake = meta.skewed != 0;
  dl.xl = dl.snake && (gridDim.x & 7) == 0;
  dl.G = dl.xl ? (int)(gridDim.x >> 3) : (int)gridDim.x;   // the snake runs over the XCD's workgroups
  dl.w = dl.xl ? (int)(blockIdx.x >> 3) : (int)blockIdx.x;
  dl.tpe = tpe;
  dl.n = dl.xl ? meta.xe[h] - meta.xb[h] : tpe * (dl.snake ? meta.cpre[E] : E);
  dl.sp = xcd_span(dl.n);
  return dl;
}

// Cost-weighted deal of two kinds of items within each XCD block.  The
// kind whose items cost more is dealt round-robin as in xcd_span, so the
// first r workgroups of the XCD get one item more than the others.  The
// other kind fills up: in fH full rounds every workgroup takes one item
// (round-robin, as xcd_span), where fH is what the loaded workgroups can take
// within the XCD's mean cost; the rest goes round-robin to the others only.
// Within a round the XCD's workgroups take consecutive items, so operands
// shared by neighbouring tiles stay in L2 together.  Plain round-robin of
// both kinds gives the extra items of both to the same low-index workgroups.
// Costs are in k-tile units.
__device__ __forceinline__ void cost_deal(int n0, int c0, int n1, int c1, Span& s0, Span& s1) {
  const bool sw = c1 > c0;
  const int nA = sw ? n1 : n0, cA = sw ? c1 : c0, nB = sw ? n0 : n1, cB = sw ? c0 : c1;
  const Span sa = xcd_span(nA);
  Span sb = xcd_span(nB);
  const int G = gridDim.x;
  const bool x8 = (G & 7) == 0;
  const int P = x8 ? G >> 3 : G, j = x8 ? (int)(blockIdx.x >> 3) : (int)blockIdx.x;
  const int x = x8 ? (int)(blockIdx.x & 7) : 0, nxcd = x8 ? 8 : 1;
  const int cha = (nA + nxcd - 1) / nxcd, chb = (nB + nxcd - 1) / nxcd;
  const int alo = min(nA, x * cha), ahi = min(nA, alo + cha);
  const int blo = min(nB, x * chb), bhi = min(nB, blo + chb);
  const int NA = ahi - alo, NB = bhi - blo;
  const int r = NA % P, q = NA / P;
  if (r > 0 && cB > 0) {
    // filler items the r loaded workgroups can take within the mean cost
    const long S = (long)NA * cA + (long)NB * cB;
    const long fh = ((S - (long)P * (q + 1) * cA) >= 0) ? (S - (long)P * (q + 1) * cA) / ((long)P * cB) : -1;
    if (fh >= 0) {
      // fH rounded down or up, whichever gives the smaller largest cost
      auto worst = [&](long fq) {
        const long rest = (long)NB - fq * P;
        return max((long)(q + 1) * cA + fq * cB, (long)q * cA + (fq + (rest + P - r - 1) / (P - r)) * cB);
      };
      long fq = min((long)NB / P, fh);
      if (fq + 1 <= (long)NB / P && worst(fq + 1) < worst(fq)) ++fq;
      // plain round-robin: workgroup 0 gets the extra item of both kinds
      const long plain = (long)(q + 1) * cA + (long)(NB / P + (NB % P > 0 ? 1 : 0)) * cB;
      if (worst(fq) < plain) {
        const int fH = (int)fq;
        sb = {blo + j, blo + fH * P, P};
        if (j >= r) {
          sb.begin2 = blo + fH * P + (j - r);
          sb.end2 = bhi;
          sb.step2 = P - r;
        }
      }
    }
  }
  s0 = sw ? sb : sa;
  s1 = sw ? sa : sb;
}

// Completes the weight-gradient tiles whose contraction was split: grads of
// tile t of expert e (an m x n block of a [M, N] gradient at g) += the
// partial tiles of chunks 1.. in chunk order; returns this thread's share of
// the tile's sum of squares.  part holds 128 x 128 fp32 tiles, row-major.
__device__ __forceinline__ float fix_split_tile(const Meta& meta, float* g, const float* part, int e, int t, int M,
                                                int N, int NT) {
  const int mt = t / NT, nt = t % NT, m0 = mt * gemm::BM, n0 = nt * gemm::BN, S = meta.nch[e];
  const int tpe = ceil_div(M, gemm::BM) * NT;
  float sq = 0.f;
  for (int idx = threadIdx.x; idx < gemm::BM * gemm::BN / 4; idx += kThreads) {
    const int r = idx / (gemm::BN / 4), c = (idx % (gemm::BN / 4)) * 4;
    if (m0 + r >= M || n0 + c >= N) continue;
    float4* gp = reinterpret_cast<float4*>(g + (long)(m0 + r) * N + n0 + c);
    float4 v = *gp;
    for (int ch = 1; ch < S; ++ch) {
      const float4 u = *reinterpret_cast<const float4*>(
          part + ((long)(meta.pbase[e] + ch - 1) * tpe + t) * (gemm::BM * gemm::BN) + r * gemm::BN + c);
      v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
    }
    *gp = v;
    sq += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  return sq;
}

__device__ __forceinline__ void trace_mark(const KParams& p, int phase, int slot) {
  if ((p.flags & 0x8u) && p.trace && threadIdx.x == 0)
    p.trace[((size_t)blockIdx.x * kPhases + phase) * 3 + slot] = wall_clock64();
}

// Stages columns [c0, c0 + dc) of W_r's expert groups [EG0, EG0 + NG) into
// LDS in the order the router's segments read them (see router_segment_sums).
// VEC: E is a multiple of 4, so a group is one 16-byte load.
template <bool VEC, int EGT, int EG0>
__device__ __forceinline__ void stage_router_rows(const KParams& p, float4* wl, int c0, int dc, int NG, int S) {
  const int tid = threadIdx.x, d = p.d, E = p.E;
  const int lg = __builtin_ctz(8 * S);   // log2 of the piece width 8 S
  // two rows per step while a pass stages at most 4 groups, else one (the
  // loads of a step stay within the register budget)
  constexpr int R = EGT <= 4 ? 2 : 1;
  for (int cb = 0; cb < dc; cb += R * kThreads) {
    float4 w[R][EGT];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float* row = p.params + (long)min(c0 + cb + r * kThreads + tid, d - 1) * E + EG0 * 4;
#pragma unroll
      for (int g = 0; g < EGT; ++g) {
        if (VEC) {
          // groups past NG read group NG - 1 again; they are never stored
          w[r][g] = *reinterpret_cast<const float4*>(row + 4 * min(g, NG - 1));
        } else {
          // expert e = 4 (EG0 + g) + t; e < E for t = 0 in every staged group
          const int e = (EG0 + min(g, NG - 1)) * 4;
          float v[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float a = row[min(e + t, E - 1) - EG0 * 4];
            v[t] = e + t < E ? a : 0.f;
          }
          w[r][g] = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int cl = cb + r * kThreads + tid;
      if (cl < dc) {
        const bool live = c0 + cl < d;   // columns past d are zeros
        const int i = cl >> lg, s = (cl >> 3) & (S - 1), j = cl & 7;
        float4* dst = wl + (i * 8 + j) * NG * S + s;
#pragma unroll
        for (int g = 0; g < EGT; ++g)
          if (g < NG)
            dst[g * S] = make_float4(live ? w[r][g].x : 0.f, live ? w[r][g].y : 0.f, live ? w[r][g].z : 0.f,
                                     live ? w[r][g].w : 0.f);
      }
    }
  }
}

// Partial router logits of TL tokens over one column segment (see the
// router phase): acc[u][e] = sum over the segment's columns c of
// x[tok + u][c] W_r[c][e], for the EGT groups of 4 experts from group EG0 on
// (padded experts read zero weights).  Each W_r value read from LDS serves
// all TL tokens.  W_r goes through LDS chunk by chunk; the tokens' 8-column
// pieces are loaded PG at a time, one group ahead of the group being
// multiplied.
template <typename T, int EGT, int EG0, int TL, int PG>
__device__ __forceinline__ void router_segment_sums(const KParams& p, const T* x, float4* wl,
                                                    float (&acc)[TL][kMaxExperts], int tok, int nmine, int s_me,
                                                    int S, int wbudget, int EG) {
  const int tid = threadIdx.x, d = p.d, E = p.E;
#pragma unroll
  for (int u = 0; u < TL; ++u)
#pragma unroll
    for (int e = 4 * EG0; e < 4 * (EG0 + EGT); ++e) acc[u][e] = 0.f;
  // only this pass's expert groups are staged, so a chunk holds as many
  // columns as the budget allows for NG groups
  const int NG = min(EGT, EG - EG0);
  if (NG <= 0) return;
  int DC = (wbudget / (NG * 16)) / (8 * S) * (8 * S);
  DC = min(max(DC, 8 * S), ceil_div(d, 8 * S) * (8 * S));
  for (int c0 = 0; c0 < d; c0 += DC) {
    const int dc = min(DC, ceil_div(d - c0, 8 * S) * (8 * S));
    const int ni = dc / (8 * S);
    auto load_group = [&](int i0, Raw8<T> (&xr)[TL][PG]) {
#pragma unroll
      for (int u = 0; u < TL; ++u)
#pragma unroll
        for (int v = 0; v < PG; ++v) {
          const int c = c0 + (i0 + v) * 8 * S + 8 * s_me;
          xr[u][v] = Raw8<T>{};
          if (u < nmine && i0 + v < ni && c < d) xr[u][v] = ldr8(x + (long)(tok + u) * d + c);
        }
    };
    // the tokens' first pieces are in flight while W_r is staged
    Raw8<T> xa[TL][PG], xb[TL][PG];
    load_group(0, xa);
    __syncthreads();
    // W_r chunk -> LDS, one column's NG groups (a contiguous row segment of
    // W_r) per thread and step, two steps' loads in flight before their
    // stores.  Column cl goes to piece cl / 8S, segment (cl / 8) % S, row
    // cl % 8 of the piece; 8S is a power of two, so these are shifts and
    // masks.  Columns past d read a clamped row and store zeros.
    if ((E & 3) == 0) stage_router_rows<true, EGT, EG0>(p, wl, c0, dc, NG, S);
    else stage_router_rows<false, EGT, EG0>(p, wl, c0, dc, NG, S);
    __syncthreads();
    for (int i0 = 0; i0 < ni; i0 += PG) {
      load_group(i0 + PG, xb);
#pragma unroll
      for (int v = 0; v < PG; ++v) {
        if (i0 + v < ni) {
          F8 xv[TL];
#pragma unroll
          for (int u = 0; u < TL; ++u) xv[u] = cvt8(xa[u][v]);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            // with several tokens per lane, W_r reads are not hoisted across
            // rows j, so the reads in flight do not outgrow the register file
            if (TL > 1) asm volatile("" ::: "memory");
            const float4* wr = wl + ((i0 + v) * 8 + j) * NG * S + s_me;
            float4 w[EGT];
#pragma unroll
            for (int eg = 0; eg < EGT; ++eg) w[eg] = eg < NG ? wr[eg * S] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int u = 0; u < TL; ++u)
#pragma unroll
              for (int eg = 0; eg < EGT; ++eg) {
                acc[u][(EG0 + eg) * 4 + 0] += xv[u].v[j] * w[eg].x;
                acc[u][(EG0 + eg) * 4 + 1] += xv[u].v[j] * w[eg].y;
                acc[u][(EG0 + eg) * 4 + 2] += xv[u].v[j] * w[eg].z;
                acc[u][(EG0 + eg) * 4 + 3] += xv[u].v[j] * w[eg].w;
              }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < TL; ++u)
#pragma unroll
        for (int v = 0; v < PG; ++v) xa[u][v] = xb[u][v];
    }
  }
}

// Sums the S segment partials of experts [4 EG0, 4 (EG0 + EGT)) of each token
// of the block into zacc, in segment order: every thread parks its partial
// sums in LDS (rows of the pass's experts + 4 floats, so the 16-byte writes of
// a wave spread over the banks), then one thread per (token, expert) adds them
// up.  The staged W_r chunk is dead by now; its space holds the partials.
// With one segment per token, or too little LDS, the segments are combined by
// a butterfly over adjacent lanes instead (the same order of additions for
// every token).  Thread (t_me, s_me) holds tokens t_me TL + u.
template <int EG0, int EGT, int TL>
__device__ __forceinline__ void router_reduce(float (&acc)[TL][kMaxExperts], float* zacc, float4* wl, int E, int EP,
                                              int S, int nb, int t_me, int s_me, int wbudget) {
  const int tid = threadIdx.x;
  const int e0 = 4 * EG0, ne = min(E, 4 * (EG0 + EGT)) - e0;
  const int RW = ceil_div(ne, 4) * 4 + 4;
  if (S > 1 && kThreads * TL * RW * 4 <= wbudget) {
    float* part = reinterpret_cast<float*>(wl);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < TL; ++u)
#pragma unroll
      for (int eg = 0; eg < EGT; ++eg)
        if (eg * 4 < ne)
          *reinterpret_cast<float4*>(part + ((t_me * TL + u) * S + s_me) * RW + eg * 4) =
              make_float4(acc[u][e0 + eg * 4], acc[u][e0 + eg * 4 + 1], acc[u][e0 + eg * 4 + 2],
                          acc[u][e0 + eg * 4 + 3]);
    __syncthreads();
    for (int o = tid; o < nb * ne; o += kThreads) {
      const int tk = o / ne, e = o % ne;
      const float* src = part + tk * S * RW + e;
      float s = 0.f;
      // the reads of 16 segments are in flight together; the sum keeps
      // segment order
      for (int sg0 = 0; sg0 < S; sg0 += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = src[min(sg0 + u, S - 1) * RW];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (sg0 + u < S) s += v[u];
      }
      zacc[tk * EP + e0 + e] = s;
    }
  } else {
#pragma unroll
    for (int u = 0; u < TL; ++u)
#pragma unroll
      for (int e = 0; e < 4 * EGT; ++e) {
        if (e < ne) {
          for (int m = S >> 1; m >= 1; m >>= 1) acc[u][e0 + e] += __shfl_xor(acc[u][e0 + e], m, 64);
        }
      }
    __syncthreads();
    if (s_me == 0) {
#pragma unroll
      for (int u = 0; u < TL; ++u)
        if (t_me * TL + u < nb) {
#pragma unroll
          for (int e = 0; e < 4 * EGT; ++e)
            if (e < ne) zacc[(t_me * TL + u) * EP + e0 + e] = acc[u][e0 + e];
        }
    }
  }
  __syncthreads();
}

// Router logits of a block of nb tokens into zacc ([nb][EP]); thread
// (t_me, s_me) covers tokens b0 + t_me TL + u of column segment s_me.
template <typename T, int OCC, int TL>
__device__ __forceinline__ void router_block(const KParams& p, const T* x, float4* wl, float* zacc, int b0, int nb,
                                             int t_me, int s_me, int S, int EG, int EP, int wbudget) {
  const int E = p.E;
  const int tok = b0 + t_me * TL;
  const int nmine = min(TL, max(0, nb - t_me * TL));
  // pieces per load group: fewer with more tokens per lane, and fewer with
  // half the register file
  constexpr int PG = TL == 1 ? 4 : 2;
  float acc[TL][kMaxExperts];
  if (EG <= 4) {
    router_segment_sums<T, 4, 0, TL, PG>(p, x, wl, acc, tok, nmine, s_me, S, wbudget, EG);
    router_reduce<0, 4, TL>(acc, zacc, wl, E, EP, S, nb, t_me, s_me, wbudget);
  } else if constexpr (TL == 1 && OCC == 1) {
    // more than 16 experts: two passes over the columns, 8 expert groups
    // each (one pass over all 64 would not fit the register file)
    router_segment_sums<T, 8, 0, 1, 4>(p, x, wl, acc, tok, nmine, s_me, S, wbudget, EG);
    router_segment_sums<T, 8, 8, 1, 4>(p, x, wl, acc, tok, nmine, s_me, S, wbudget, EG);
    router_reduce<0, 16, 1>(acc, zacc, wl, E, EP, S, nb, t_me, s_me, wbudget);
  } else if constexpr (TL == 1) {
    // with half the registers: passes of 16 experts, each summed over the
    // segments before the next one starts
    router_segment_sums<T, 4, 0, 1, 4>(p, x, wl, acc, tok, nmine, s_me, S, wbudget, EG);
    router_reduce<0, 4, 1>(acc, zacc, wl, E, EP, S, nb, t_me, s_me, wbudget);
    router_segment_sums<T, 4, 4, 1, 4>(p, x, wl, acc, tok, nmine, s_me, S, wbudget, EG);
    router_reduce<4, 4, 1>(acc, zacc, wl, E, EP, S, nb, t_me, s_me, wbudget);
    if (EG > 8) {
      router_segment_sums<T, 4, 8, 1, 4>(p, x, wl, acc, tok, nmine, s_me, S, wbudget, EG);
      router_reduce<8, 4, 1>(acc, zacc, wl, E, EP, S, nb, t_me, s_me, wbudget);
    }
    if (EG > 12) {
      router_segment_sums<T, 4, 12, 1, 4>(p, x, wl, acc, tok, nmine, s_me, S, wbudget, EG);
      router_reduce<12, 4, 1>(acc, zacc, wl, E, EP, S, nb, t_me, s_me, wbudget);
    }
  }
}

// Router logits of tokens [b0, b0 + nb) on the matrix cores, for d a multiple
// of 128 up to kRouterMfmaMaxD: zacc[t][e] = sum_c x[b0 + t][c] W_r[c][e] in
// fp32 with v_mfma_f32_16x16x4_f32, 16 tokens x 16 experts per product (token
// tiles of 16 rows, expert tiles of 16 columns).  The contraction over the d
// columns is split 16 ways: wave w and lane group g = lane / 16 own the
// L = d / 16 consecutive columns from (4 w + g) L, and each product takes one
// column of every lane group.  A lane supplies the x value of token row
// lane % 16 and the W_r value of expert column lane % 16, both read straight
// from global memory (each wave reads only its own quarter of W_r): all of a
// lane's W_r values of an expert tile are requested at once, and the x values
// of the next token tile while this tile is multiplied, so a block costs about
// one memory round trip per expert tile.  The four waves' partial tiles go
// through LDS (part, [4][ntt * 16][EP]) and are added in wave order into zacc
// ([ntt * 16][EP]).
constexpr int kRouterMfmaMaxD = 1024;
template <typename T>
__device__ __forceinline__ void router_mfma_block(const KParams& p, const T* x, float* zacc, float* part, int b0,
                                                  int nb, int EP) {
  constexpr int LM = kRouterMfmaMaxD / 16;   // columns per lane group at most
  constexpr int NQ = LM / 8;                 // 8-column pieces per lane group at most
  typedef float f4v __attribute__((ext_vector_type(4)));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int d = p.d, E = p.E;
  const int L = d >> 4, nq = L >> 3;         // columns and 8-column pieces per lane group
  const int i = lane & 15, g = lane >> 4;
  const int kb = (wave * 4 + g) * L;         // first column of this lane group
  const int ntt = (nb + 15) >> 4, net = (E + 15) >> 4;
  const int TPB = ntt * 16;                  // token rows of the partial tiles
  // the x pieces of token row i of tile tt (rows past nb read the last token,
  // pieces past L the last piece; neither is used)
  auto load_x = [&](int tt, Raw8<T> (&xr)[NQ]) {
    const T* row = x + (long)(b0 + min(tt * 16 + i, nb - 1)) * d + kb;
#pragma unroll
    for (int q = 0; q < NQ; ++q) xr[q] = ldr8(row + 8 * min(q, nq - 1));
  };
  Raw8<T> xa[NQ], xb[NQ];
  for (int et = 0; et < net; ++et) {
    const int e = et * 16 + i;                // expert column of this lane
    const bool ein = e < E;
    const float* wcol = p.params + min(e, E - 1) + (long)kb * E;
    float w[LM];
#pragma unroll
    for (int m = 0; m < LM; ++m) w[m] = wcol[(long)min(m, L - 1) * E];
    if (!ein) {
#pragma unroll
      for (int m = 0; m < LM; ++m) w[m] = 0.f;
    }
    if (et == 0) load_x(0, xa);
    for (int tt = 0; tt < ntt; ++tt) {
      // x of the next tile (or, for the last, of the first tile of the next
      // expert tile) in flight while this one is multiplied
      const bool last = tt + 1 == ntt;
      if (!last || et + 1 < net) load_x(last ? 0 : tt + 1, xb);
      f4v c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if (q < nq) {
          const F8 xf = cvt8(xa[q]);
#pragma unroll
          for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(xf.v[s], w[q * 8 + s], c, 0, 0, 0);
        }
      }
      // partial tile of this wave: the lane holds rows 4 (lane / 16) + r of
      // column lane % 16
      if (e < EP) {
        float* dst = part + ((long)wave * TPB + tt * 16 + 4 * g) * EP + e;
        dst[0] = c.x;
        dst[EP] = c.y;
        dst[2 * EP] = c.z;
        dst[3 * EP] = c.w;
      }
#pragma unroll
      for (int q = 0; q < NQ; ++q) xa[q] = xb[q];
    }
  }
  __syncthreads();
  for (int o = tid; o < nb * EP; o += kThreads) {
    const int t = o / EP, ee = o - t * EP;
    const float* src = part + (long)t * EP + ee;
    zacc[o] = ((src[0] + src[(long)TPB * EP]) + src[2L * TPB * EP]) + src[3L * TPB * EP];
  }
  __syncthreads();
}

// ===========================================================================
// P0: weight-copy refresh, W_r^T, router logits + token_topk + gates + histogram
// ===========================================================================
template <typename T, int OCC>
__device__ __forceinline__ void phase_route(const KParams& p, char* smem, Meta& meta) {
  const int tid = threadIdx.x;
  const int G = gridDim.x, lwg = logical_wg();
  const int d = p.d, E = p.E, k = p.k;

  // bf16 copy of W1 | W2 from the fp32 master weights
  if ((p.flags & 0x4u) && p.shadow) {
    const long nw = 2L * E * d * p.f;
    const float* src = p.params + (long)d * E;
    for (long i = ((long)lwg * kThreads + tid) * 8; i < nw; i += (long)G * kThreads * 8)
      st8(p.shadow + i, ld8(src + i));
  }
  // W_r^T, read by the input-gradient phase after AdamW may have changed W_r
  for (int i = lwg * kThreads + tid; i < d * E; i += G * kThreads) {
    const int c = i / E, e = i % E;
    p.wrt[(long)e * d + c] = p.params[i];
  }

  int* hist = reinterpret_cast<int*>(smem);                  // [64]
  int EP = 1;
  while (EP < E) EP <<= 1;
  const int TPI = kThreads / EP;          // tokens per top-k pass
  const int per = ceil_div(p.T, G);
  const int t_lo = min(p.T, lwg * per), t_hi = min(p.T, t_lo + per);
  if (tid < kMaxExperts) hist[tid] = 0;
  const int e_me = tid % EP, slot = tid / EP;
  const T* x = reinterpret_cast<const T*>(p.x);

  constexpr int kScratch = scratch_bytes(OCC);
  constexpr int kSelBytes = kThreads * kMaxTopK * 4;   // the top-k selections of one pass, at the end of the scratch
  float* zacc = reinterpret_cast<float*>(smem + 256);   // [TP][EP] logits of a block
  // token_topk over each group of EP lanes for the logits of tokens
  // [b0, b0 + nb) in zacc ([nb][EP]), TPI tokens per pass.  Each lane of a
  // token writes its biased logit back (non-finite ones become -inf and set
  // an error bit), then counts the experts that come before it (a larger
  // logit, or an equal one and a lower index): that count is its rank, and
  // ranks below k are the selection, in order.  The selected logits go to
  // sel ([TPI][kMaxTopK]) so every selected lane forms the softmax
  // denominator over them in rank order.
  float* sel = reinterpret_cast<float*>(smem + kScratch - kSelBytes);
  auto topk_block = [&](int b0, int nb) {
    for (int g0 = 0; g0 < nb; g0 += TPI) {
      const int tok = b0 + g0 + slot;
      const bool active = (g0 + slot) < nb && e_me < E;
      float* zr = zacc + (g0 + slot) * EP;
      float z = -INFINITY;
      if (active) {
        z = zr[e_me];
        if (p.bias) z += p.bias[e_me];
        if (p.dbg_logits) p.dbg_logits[(long)tok * E + e_me] = z;
        if (!(z == z) || z == INFINITY || z == -INFINITY) {   // NaN or infinite: device error
          __hip_atomic_fetch_or(p.ctrl.status, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          z = -INFINITY;
        }
        zr[e_me] = z;
      }
      __syncthreads();
      int rank = kMaxExperts;
      if (active) {
        rank = 0;
        if ((EP & 3) == 0) {
          for (int e4 = 0; e4 < E; e4 += 4) {
            const float4 o = *reinterpret_cast<const float4*>(zr + e4);
            rank += (o.x > z) || (o.x == z && e4 < e_me);
            if (e4 + 1 < E) rank += (o.y > z) || (o.y == z && e4 + 1 < e_me);
            if (e4 + 2 < E) rank += (o.z > z) || (o.z == z && e4 + 2 < e_me);
            if (e4 + 3 < E) rank += (o.w > z) || (o.w == z && e4 + 3 < e_me);
          }
        } else {
          for (int e2 = 0; e2 < E; ++e2) {
            const float o = zr[e2];
            rank += (o > z) || (o == z && e2 < e_me);
          }
        }
        if (rank < k) sel[slot * kMaxTopK + rank] = z;
      }
      __syncthreads();
      if (rank < k) {
        const float* zs = sel + slot * kMaxTopK;
        const float z0 = zs[0];
        float den = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j)
          if (j < k) den += expf(zs[j] - z0);
        const float gj = expf(z - z0) / den;
        const int q = tok * k + rank;
        p.idx[q] = e_me;
        p.gate[q] = gj;
        if (p.dbg_idx) p.dbg_idx[q] = e_me;
        if (p.dbg_gate) p.dbg_gate[q] = gj;
        atomicAdd(&hist[e_me], 1);
      }
      __syncthreads();
    }
  };

  if ((d & 127) == 0 && d <= kRouterMfmaMaxD) {
    // matrix-core path: blocks of up to 4 token tiles of 16, as many as the
    // partial tiles, zacc, the histogram and the selections leave room for.
    // Its own loop, so the other path's loop invariants are not computed
    // (and spilled) here.
    int ntt = min(4, ceil_div(t_hi - t_lo, 16));
    while (ntt > 1 && 256 + 5 * 16 * ntt * EP * 4 + kSelBytes > kScratch) --ntt;
    const int TP = 16 * ntt;
    float* part = zacc + TP * EP;   // [4][TP][EP] partial tiles
    for (int b0 = t_lo; b0 < t_hi; b0 += TP) {
      const int nb = min(TP, t_hi - b0);
      router_mfma_block<T>(p, x, zacc, part, b0, nb, EP);
      topk_block(b0, nb);
    }
  } else {
    // Router logits, TP tokens per pass, each split over S column segments
    // (TP * S / TL <= 256 threads, S a power of two <= 64 so a token's segments are
    // adjacent lanes of one wave).  Segment s of a token owns the 8-column
    // pieces 8s, 8s + 8S, 8s + 16S, ... and keeps all E partial sums in
    // registers; W_r is staged in LDS in the order the segments read it (for
    // each piece index i, row j of the piece and 4-expert group eg, the S
    // segments' float4s side by side), so the reads of one wave are either
    // distinct consecutive 16-byte words or broadcasts.
    // The logits of a block live in LDS (zacc, [TP][EP]) within a quarter of the
    // scratch; a larger token range takes several blocks.
    // With 16 or more tokens per pass and at most 16 experts, each lane works
    // on TL tokens (4 with one workgroup per CU, 2 with half the register
    // file), so every W_r value it reads from LDS serves TL tokens.
    int TP = 1;
    while (TP < min(t_hi - t_lo, 4 * kThreads) && 2 * TP * EP * 4 <= kScratch / 4) TP <<= 1;
    const int EG = (E + 3) / 4;
    constexpr int kTL = OCC == 1 ? 4 : 2;
    const int TL = (TP >= 16 && EG <= 4) ? kTL : 1;
    TP = min(TP, TL * kThreads);
    int S = min(64, kThreads * TL / TP);
    while (S > 1 && 8 * S > d) S >>= 1;
    float4* wl = reinterpret_cast<float4*>(smem + 256 + TP * EP * 4);           // staged W_r chunk
    // (the reads of padded expert groups may run up to 16 * S float4 past the chunk)
    const int wbudget = kScratch - 256 - TP * EP * 4 - 16 * 64 * 16;
    // a chunk holds at least one 8-column piece per segment for every expert
    // group a pass stages (all EG groups in one pass up to 16 experts, else 8
    // groups per pass with a whole register file, 4 with half of it; 8 * 8 * 16
    // bytes always fit, so this ends with chunks of at least 8 S columns)
    const int NGmax = EG <= 4 ? EG : (OCC == 1 ? 8 : 4);
    while (S > 1 && 8 * S * NGmax * 16 > wbudget) S >>= 1;
    const int t_me = tid / S, s_me = tid % S;

    for (int b0 = t_lo; b0 < t_hi; b0 += TP) {
      const int nb = min(TP, t_hi - b0);
      if (TL > 1) router_block<T, OCC, kTL>(p, x, wl, zacc, b0, nb, t_me, s_me, S, EG, EP, wbudget);
      else router_block<T, OCC, 1>(p, x, wl, zacc, b0, nb, t_me, s_me, S, EG, EP, wbudget);
      topk_block(b0, nb);
    }
  }
  __syncthreads();
  if (tid < E) p.hist[(long)lwg * E + tid] = hist[tid];
}

// ===========================================================================
// P1: route_order -- offsets and a stable scatter of the flat ids by expert
// ===========================================================================
template <typename T>
__device__ __forceinline__ void phase_order(const KParams& p, char* smem, Meta& meta, bool skip_scatter) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = gridDim.x, lwg = logical_wg();
  const int E = p.E, k = p.k;
  int EP = 1, EB = 0;
  while (EP < E) { EP <<= 1; ++EB; }
  const int parts = kThreads / EP;

  int* sp = reinterpret_cast<int*>(smem);             // [parts][EP] prefix (w < lwg)
  int* st = sp + kThreads;                            // [parts][EP] totals
  int* base = st + kThreads;                          // [EP]
  int* cw = base + kMaxExperts;                       // [kWaves][EP]
  int* posl = cw + kWaves * kMaxExperts;              // [kThreads] sorted positions of this block
  if (p.flags & 0x10000u)   // readiness counters of this launch, zero before GEMM 1 starts
    for (int i = lwg * kThreads + tid; i < p.nrb; i += G * kThreads) p.ready[i] = 0;
  {
    // 32 rows per thread in flight at once: with up to 16 experts and 512
    // workgroups that is every row in one round of (L2-missing) loads
    const int e = tid % EP, part = tid / EP;
    int pre = 0, tot = 0;
    if (e < E) {
      for (int w0 = part; w0 < G; w0 += parts * 32) {
        int h[32];
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          const int w = w0 + u * parts;
          h[u] = (w < G) ? p.hist[(long)w * E + e] : 0;
        }
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          tot += h[u];
          if (w0 + u * parts < lwg) pre += h[u];
        }
      }
    }
    sp[tid] = pre;
    st[tid] = tot;
  }
  __syncthreads();
  if (tid < EP) {
    int pre = 0, tot = 0;
    for (int q = 0; q < parts; ++q) {
      pre += sp[q * EP + tid];
      tot += st[q * EP + tid];
    }
    sp[tid] = pre;       // reuse row 0
    st[tid] = tot;
  }
  __syncthreads();
  if (tid == 0) {
    int o = 0, mo = 0;
    for (int e = 0; e < E; ++e) {
      meta.cnt[e] = st[e];
      meta.wcnt[e] = st[e];
      meta.off[e] = o;
      meta.moff[e] = mo;
      o += st[e];
      mo += ceil_div(st[e], gemm::BM);
    }
    meta.off[E] = o;
    meta.moff[E] = mo;
  }
  __syncthreads();
  if (p.defer) {
    // the rows the weight-gradient products contract over (wcnt, this
    // launch's own otherwise): with deferred weight gradients this launch's
    // counts and offsets go to its slot, and the applying launch adds the
    // earlier slots' (written by earlier launches)
    if (tid < E) {
      int w = meta.cnt[tid];
      if (lwg == 0) {
        p.slot_cnt[p.slot * E + tid] = meta.cnt[tid];
        p.slot_off[p.slot * E + tid] = meta.off[tid];
      }
      if (p.defer_final)
        for (int s = 0; s < p.slot; ++s) w += p.slot_cnt[s * E + tid];
      else
        w = 0;
      meta.wcnt[tid] = w;
    }
    __syncthreads();
  }
  if (tid < E) {
    // rank of this expert by row count, for dealing the weight-gradient tiles
    const int c = meta.wcnt[tid];
    int r = 0;
    for (int e = 0; e < E; ++e) r += (meta.wcnt[e] > c) || (meta.wcnt[e] == c && e < tid);
    meta.ord[r] = tid;
  }
  if (tid == 0) {
    int mx = 0, tot = 0;
    for (int e = 0; e < E; ++e) {
      mx = max(mx, meta.wcnt[e]);
      tot += meta.wcnt[e];
    }
    meta.wtot = tot;
    // The applying launch of deferred weight gradients contracts over every
    // slot's rows: its contractions are long and few per workgroup, so it
    // always splits them, in chunks of the mean rows per expert (at most E
    // extra chunks; half the mean measured 0.6% slower on the Zipf workload,
    // its extra partial tiles costing more than the finer deal saved);
    // otherwise chunks of twice the mean under skew (at most E/2 extra).
    const bool dfin = p.defer && p.defer_final;
    meta.skewed = dfin ? tot > 0 : (long)mx * E > 2L * tot;
    int kc = 64 * max(1, ceil_div(ceil_div(ceil_div(2 * tot, max(E, 1)), dfin ? 2 : 1), 64));
    // never more extra chunks than the partial-tile buffers hold (the rule
    // above stays within them; this keeps any other rule inside too)
    for (;;) {
      int extra = 0;
      for (int e = 0; e < E; ++e) extra += meta.skewed ? max(1, ceil_div(meta.wcnt[e], kc)) - 1 : 0;
      if (extra <= p.wpart_sets) break;
      kc *= 2;
    }
    meta.kc = kc;
    int pb = 0, ns = 0;
    for (int e = 0; e < E; ++e) {
      const int n = meta.skewed ? max(1, ceil_div(meta.wcnt[e], kc)) : 1;
      meta.nch[e] = n;
      meta.pbase[e] = pb;
      pb += n - 1;
      if (n > 1) meta.splitlist[ns++] = e;
    }
    meta.nsplit = ns;
  }
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int r = 0; r < E; ++r) {
      meta.cpre[r] = s;
      s += meta.nch[meta.ord[r]];
    }
    meta.cpre[E] = s;
  }
  __syncthreads();
  if (meta.skewed && (G & 7) == 0) {
    // (expert, chunk) units of the weight-gradient products, ranked by their
    // rows, longest first (ties: expert order, then chunk).  A unit's tiles
    // cost kWTileFixed[phase] + its k-tiles each; XCD x takes the tiles whose
    // cost midpoint lies in [x C / 8, (x + 1) C / 8) of the total cost C, in
    // that order, once per weight-gradient phase.  Every workgroup computes the
    // same splits and keeps its own ranges.
    int* ucost = posl + kThreads;            // [kThreads] unit rows, in expert-rank order
    int* uid = ucost + kThreads;             // [kThreads] the units
    int* scost = uid + kThreads;             // [kThreads] rows, longest first
    int* suid = scost + kThreads;            // [kThreads] units, longest first
    const int nu = meta.cpre[E];             // units: the chunks of every expert
    if (tid < E) {
      const int e = meta.ord[tid];
      for (int c = 0; c < meta.nch[e]; ++c) {
        ucost[meta.cpre[tid] + c] = meta.nch[e] > 1 ? min(meta.kc, meta.wcnt[e] - c * meta.kc) : meta.wcnt[e];
        uid[meta.cpre[tid] + c] = e | (c << 8);
      }
    }
    __syncthreads();
    if (tid < nu) {
      int rank = 0;
      for (int v = 0; v < nu; ++v) rank += (ucost[v] > ucost[tid]) || (ucost[v] == ucost[tid] && v < tid);
      scost[rank] = ucost[tid];
      suid[rank] = uid[tid];
    }
    __syncthreads();
    if (tid < nu) meta.xunit[tid] = suid[tid];
    // one thread per unit: its cost in both phases, the cost of the units
    // before it, and how many of its tiles lie below the XCD's two bounds
    // (summed in LDS)
    long* upre = reinterpret_cast<long*>(suid + kThreads);   // [2][kThreads]
    int* cntx = reinterpret_cast<int*>(upre + 2 * kThreads);  // [2][2]
    const long tpe = (long)ceil_div(p.f, gemm::BM) * ceil_div(p.d, gemm::BN);
    const int x = (int)(blockIdx.x & 7);
    const long kt = tid < nu ? ceil_div(scost[tid], 64) : 0;
    if (tid < nu) {
      upre[tid] = tpe * (kWTileFixed[0] + kt);
      upre[kThreads + tid] = tpe * (kWTileFixed[1] + kt);
    }
    if (tid < 4) cntx[tid] = 0;
    __syncthreads();
    if (tid < nu) {
#pragma unroll
      for (int ph = 0; ph < 2; ++ph) {
        const long uc = kWTileFixed[ph] + kt;
        long pre = 0, total = 0;
        for (int i = 0; i < nu; ++i) {
          const long ci = upre[ph * kThreads + i];
          pre += i < tid ? ci : 0;
          total += ci;
        }
        const long first = 8 * pre + 4 * uc;   // 8 x the midpoint of the unit's first tile
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const long lim = (long)(x + hh) * total;
          // every tile below the bound, none, or (one unit per bound) a division
          if (lim > first + 8 * uc * (tpe - 1)) atomicAdd(&cntx[2 * ph + hh], (int)tpe);
          else if (lim > first) atomicAdd(&cntx[2 * ph + hh], (int)((lim - first - 1) / (8 * uc) + 1));
        }
      }
    }
    __syncthreads();
    if (tid == 0) {
      meta.xb[0] = cntx[0];
      meta.xe[0] = cntx[1];
      meta.xb[1] = cntx[2];
      meta.xe[1] = cntx[3];
      meta.nxu = nu;
    }
    __syncthreads();
  }
  if (tid < E) base[tid] = meta.off[tid] + sp[tid];
  if (lwg == 0 && tid < E && p.dbg_counts) p.dbg_counts[tid] = meta.cnt[tid];
  if (skip_scatter) return;

  const int per = ceil_div(p.T, G);
  const int t_lo = min(p.T, lwg * per), t_hi = min(p.T, t_lo + per);
  const int q_lo = t_lo * k, q_hi = t_hi * k;
  for (int q0 = q_lo; q0 < q_hi; q0 += kThreads) {
    __syncthreads();
    for (int i = tid; i < kWaves * EP; i += kThreads) cw[i] = 0;
    __syncthreads();
    const int q = q0 + tid;
    const bool valid = q < q_hi;
    const int e = valid ? p.idx[q] : 0;
    unsigned long long mask = __ballot(valid);
    for (int b = 0; b < EB; ++b) {
      const unsigned long long bb = __ballot(valid && ((e >> b) & 1));
      mask &= ((e >> b) & 1) ? bb : ~bb;
    }
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(mask & lt);
    if (valid && (mask >> lane) == 1ull) cw[wave * EP + e] = __popcll(mask);   // highest lane of its group
    __syncthreads();
    if (valid) {
      int pos = base[e] + rank;
      for (int w = 0; w < wave; ++w) pos += cw[w * EP + e];
      p.perm[pos] = q;
      p.inv[q] = pos;
      if (p.dbg_perm) p.dbg_perm[pos] = q;
      posl[tid] = pos;
    }
    __syncthreads();
    if (sizeof(T) == 2 && !(p.flags & 0x100000u)) {
      // dispatch gather: the token row of each routed row of this block is
      // copied to its sorted position (xs, [N, d] in expert order), so the
      // expert products read contiguous rows
      const int nq = min(kThreads, q_hi - q0), d = p.d, U = d / 8;
      const uint16_t* xg = reinterpret_cast<const uint16_t*>(p.x);
      uint16_t* xs = reinterpret_cast<uint16_t*>(p.xs);
#pragma unroll 4
      for (int u = tid; u < nq * U; u += kThreads) {
        const int i = u / U, c = (u - i * U) * 8;
        *reinterpret_cast<uint4*>(xs + (long)posl[i] * d + c) =
            *reinterpret_cast<const uint4*>(xg + (long)((q0 + i) / k) * d + c);
      }
    }
    if (tid < E) {
      int s = 0;
      for (int w = 0; w < kWaves; ++w) s += cw[w * EP + tid];
      base[tid] += s;
    }
  }
}

// Expert owning global row-tile mg (moff is ascending).
__device__ __forceinline__ int expert_of_tile(const Meta& meta, int E, int mg) {
  int e = 0;
  while (e + 1 < E && meta.moff[e + 1] <= mg) ++e;
  return e;
}

template <typename T>
__device__ __forceinline__ const T* w1_ptr(const KParams& p) {
  if constexpr (sizeof(T) == 2) return reinterpret_cast<const T*>(p.shadow);
  else return reinterpret_cast<const T*>(p.params + (long)p.d * p.E);
}
template <typename T>
__device__ __forceinline__ const T* w2_ptr(const KParams& p) {
  return w1_ptr<T>(p) + (long)p.E * p.d * p.f;
}

// ===========================================================================
// P2: ragged_mm 1 + GELU.  Rows of expert e: x[perm[p]/k], p in its segment
// (bf16: read from the copy in xs).
// ===========================================================================
template <typename T, int NS>
__device__ __forceinline__ void phase_ffn1(const KParams& p, char* lds, const Meta& meta, bool publish) {
  const int G = gridDim.x, lwg = logical_wg();
  const int d = p.d, f = p.f;
  const int NT = ceil_div(f, gemm::BN);
  const int ntiles = meta.moff[p.E] * NT;
  T* act = reinterpret_cast<T*>(p.act);
  T* gp = reinterpret_cast<T*>(p.gp);
  const Span sp = xcd_span(ntiles);
  for (int tI = sp.begin; tI < sp.end; tI += sp.step) {
    const int mg = tI / NT, nt = tI % NT;
    const int e = expert_of_tile(meta, p.E, mg);
    const int m0 = (mg - meta.moff[e]) * gemm::BM;
    const int p0 = meta.off[e] + m0;
    const int mrows = min(gemm::BM, meta.cnt[e] - m0);
    // bf16: the gathered rows (xs, contiguous); fp32: token rows through perm
    const gemm::Operand A = sizeof(T) == 2
                                ? gemm::Operand{reinterpret_cast<const char*>(p.xs), d, nullptr, 1, p0, mrows, d, 0}
                                : gemm::Operand{reinterpret_cast<const char*>(p.x), d, p.perm, p.k, p0, mrows, d, 0};
    gemm::Operand B{reinterpret_cast<const char*>(w1_ptr<T>(p) + (long)e * d * f), f, nullptr, 1, 0, d, f,
                    nt * gemm::BN};
    const int n0 = nt * gemm::BN;
    auto epi = [&](int r, int c, const float (&h)[8]) {
      if (r < mrows && n0 + c < f) {
        const long o = (long)(p0 + r) * f + n0 + c;
        if (p.recompute) {   // memory rule: keep H only
          F8 hv;
#pragma unroll
          for (int q = 0; q < 8; ++q) hv.v[q] = h[q];
          st8s(act + o, hv, p.nt_stores);
          return;
        }
        F8 a, da;
#pragma unroll
        for (int q = 0; q < 8; ++q) gelu_and_grad(h[q], a.v[q], da.v[q]);
        st8s(act + o, a, p.nt_stores);
        st8s(gp + o, da, p.nt_stores);
      }
    };
    gemm::tile<T, NS, false, true>(lds, A, B, d, epi);
    if (publish) {
      // every wave's stores of the tile have reached L2; one agent-scope
      // release for the workgroup (the XCD's L2 is written back), then the count
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      if (threadIdx.x == 0) {
        release_agent();
        __hip_atomic_fetch_add(p.ready + mg, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// ===========================================================================
// P3: ragged_mm 2:  O = A_e W2[e]
// ===========================================================================
// With `wait` (readiness mode), a tile first waits until every GEMM-1 column
// tile of its 128 rows is counted done, then acquires.  False if that wait
// timed out (or another workgroup gave up).
template <typename T, int NS>
__device__ __forceinline__ bool phase_ffn2(const KParams& p, char* lds, Meta& meta, bool wait) {
  const int G = gridDim.x, lwg = logical_wg();
  const int d = p.d, f = p.f;
  const int NT = ceil_div(d, gemm::BN);
  const int ntiles = meta.moff[p.E] * NT;
  const Span sp = xcd_span(ntiles);
  for (int tI = sp.begin; tI < sp.end; tI += sp.step) {
    const int mg = tI / NT, nt = tI % NT;
    if (wait) {
      if (threadIdx.x == 0) {
        const bool ok = wait_count(p.ctrl, p.ready + mg, ceil_div(f, gemm::BN));
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        meta.bar.flag = ok ? 1u : 0u;
      }
      __syncthreads();
      if (meta.bar.flag == 0u) return false;
    }
    const int e = expert_of_tile(meta, p.E, mg);
    const int m0 = (mg - meta.moff[e]) * gemm::BM;
    const int p0 = meta.off[e] + m0;
    const int mrows = min(gemm::BM, meta.cnt[e] - m0);
    gemm::Operand A{reinterpret_cast<const char*>(p.act), f, nullptr, 1, p0, mrows, f, 0};
    gemm::Operand B{reinterpret_cast<const char*>(w2_ptr<T>(p) + (long)e * f * d), d, nullptr, 1, 0, f, d,
                    nt * gemm::BN};
    const int n0 = nt * gemm::BN;
    auto epi = [&](int r, int c, const float (&v)[8]) {
      if (r < mrows && n0 + c < d) {
        F8 o;
#pragma unroll
        for (int q = 0; q < 8; ++q) o.v[q] = v[q];
        st8s(p.out + (long)(p0 + r) * d + n0 + c, o, p.nt_stores);
      }
    };
    // under the recomputation rule act holds H and the A fragments pass through GELU
    if (p.recompute) gemm::tile<T, NS, false, true, true>(lds, A, B, f, epi);
    else gemm::tile<T, NS, false, true, false>(lds, A, B, f, epi);
  }
  return true;
}

// ===========================================================================
// P4: combine, loss, dL/dO, dL/dgate -> dL/dlogit (one wave per token)
// ===========================================================================
// One token per half-wave: lane h of the half owns columns 8h.. of every
// 256-column chunk.  CP chunks of the token are loaded at once (CP * k <= 8
// row pieces of `out`), and the gates and slots of the half-wave's next token
// are loaded one token ahead, so every lane keeps several loads in flight.
// Token t goes to workgroup t % G (half-wave (t / G) % 8 of it), so every
// workgroup gets the same number of tokens to within one even when there are
// fewer tokens than half-waves.
template <typename T, int CP>
__device__ __forceinline__ float combine_tokens(const KParams& p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, hl = lane & 31;
  const int G = gridDim.x, lwg = logical_wg();
  const int d = p.d, k = p.k;
  const T* tg = reinterpret_cast<const T*>(p.t);
  T* dout = reinterpret_cast<T*>(p.dout);
  const int stride = G * kWaves * 2;
  float lsum = 0.f;
  float g[kMaxTopK], gn[kMaxTopK];
  int pos[kMaxTopK], pn[kMaxTopK];
  auto load_idx = [&](int tok, float (&gg)[kMaxTopK], int (&pp)[kMaxTopK]) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      gg[j] = 0.f;
      pp[j] = 0;
      if (j < k && tok < p.T) {
        gg[j] = p.gate[tok * k + j];
        pp[j] = p.inv[tok * k + j];
      }
    }
  };
  int base = wave * 2 * G + lwg;   // token of half-wave 0; half-wave 1 takes base + G
  load_idx(base + half * G, g, pos);
  // the loop bound is uniform over the wave (the half-wave sums need both halves)
  for (; base < p.T; base += stride) {
    const int tok = base + half * G;
    const bool live = tok < p.T;
    load_idx(tok + stride, gn, pn);
    float dg[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) dg[j] = 0.f;
    for (int c0 = 0; c0 < d; c0 += 256 * CP) {
      Raw8<T> tr[CP];
      Raw8<float> o[CP * kMaxTopK > 8 ? 8 : CP * kMaxTopK];
      constexpr int NS = CP * kMaxTopK > 8 ? 8 : CP * kMaxTopK;
#pragma unroll
      for (int ch = 0; ch < CP; ++ch) {
        const int c = c0 + ch * 256 + hl * 8;
        tr[ch] = Raw8<T>{};
        if (live && c < d) tr[ch] = ldr8(tg + (long)tok * d + c);
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int j = s / CP, ch = s % CP;
        const int c = c0 + ch * 256 + hl * 8;
        o[s] = Raw8<float>{};
        if (live && j < k && c < d) o[s] = ldr8(p.out + (long)pos[j] * d + c);
      }
      F8 y[CP];
#pragma unroll
      for (int ch = 0; ch < CP; ++ch)
#pragma unroll
        for (int q = 0; q < 8; ++q) y[ch].v[q] = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int j = s / CP, ch = s % CP;
        const F8 ov = cvt8(o[s]);
#pragma unroll
        for (int q = 0; q < 8; ++q) y[ch].v[q] += g[j] * ov.v[q];
      }
#pragma unroll
      for (int ch = 0; ch < CP; ++ch) {
        const F8 tv = cvt8(tr[ch]);
        const int c = c0 + ch * 256 + hl * 8;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float r = y[ch].v[q] - tv.v[q];
          if (live && c < d) lsum += r * r;
          y[ch].v[q] = r * p.inv_tupd;   // now dL/dy
        }
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int j = s / CP, ch = s % CP;
        const int c = c0 + ch * 256 + hl * 8;
        if (live && j < k && c < d) {
          const F8 ov = cvt8(o[s]);
          F8 w;
          float sdot = 0.f;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            w.v[q] = g[j] * y[ch].v[q];
            sdot += y[ch].v[q] * ov.v[q];
          }
          dg[j] += sdot;
          st8(dout + (long)pos[j] * d + c, w);
        }
      }
    }
    float sg = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
#pragma unroll
        for (int m = 16; m >= 1; m >>= 1) dg[j] += __shfl_xor(dg[j], m, 64);
        sg += g[j] * dg[j];
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (live && j < k && hl == j) p.dzsel[tok * k + j] = g[j] * (dg[j] - sg);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      g[j] = gn[j];
      pos[j] = pn[j];
    }
  }
  return lsum;
}

// The same for rows of at most 256 CP columns (one chunk), software-pipelined
// over the half-wave's tokens: the gates and slots are loaded two tokens
// ahead and the token and expert-output rows one token ahead, all issued
// before the current token's dO stores.  The vector-memory counter retires
// in issue order, so a load issued after a store could only be awaited
// together with the store; issued before it, the next token's rows are in
// flight while the stores drain.
template <typename T, int CP>
__device__ __forceinline__ float combine_tokens_1chunk(const KParams& p) {
  constexpr int NS = CP * kMaxTopK > 8 ? 8 : CP * kMaxTopK;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, hl = lane & 31;
  const int G = gridDim.x, lwg = logical_wg();
  const int d = p.d, k = p.k;
  const T* tg = reinterpret_cast<const T*>(p.t);
  T* dout = reinterpret_cast<T*>(p.dout);
  const int stride = G * kWaves * 2;
  float lsum = 0.f;
  float g[kMaxTopK], gn[kMaxTopK], gnn[kMaxTopK];
  int pos[kMaxTopK], pn[kMaxTopK], pnn[kMaxTopK];
  auto load_idx = [&](int tok, float (&gg)[kMaxTopK], int (&pp)[kMaxTopK]) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      gg[j] = 0.f;
      pp[j] = 0;
      if (j < k && tok < p.T) {
        gg[j] = p.gate[tok * k + j];
        pp[j] = p.inv[tok * k + j];
      }
    }
  };
  auto load_rows = [&](int tok, const int (&pp)[kMaxTopK], Raw8<T> (&tr)[CP], Raw8<float> (&o)[NS]) {
    const bool live = tok < p.T;
#pragma unroll
    for (int ch = 0; ch < CP; ++ch) {
      const int c = ch * 256 + hl * 8;
      tr[ch] = Raw8<T>{};
      if (live && c < d) tr[ch] = ldr8(tg + (long)tok * d + c);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int j = s / CP, ch = s % CP;
      const int c = ch * 256 + hl * 8;
      o[s] = Raw8<float>{};
      if (live && j < k && c < d) o[s] = ldr8(p.out + (long)pp[j] * d + c);
    }
  };
  int base = wave * 2 * G + lwg;   // token of half-wave 0; half-wave 1 takes base + G
  Raw8<T> tr[CP], trn[CP];
  Raw8<float> o[NS], on[NS];
  load_idx(base + half * G, g, pos);
  load_idx(base + half * G + stride, gn, pn);
  load_rows(base + half * G, pos, tr, o);
  // the loop bound is uniform over the wave (the half-wave sums need both halves)
  for (; base < p.T; base += stride) {
    const int tok = base + half * G;
    const bool live = tok < p.T;
    load_idx(tok + 2 * stride, gnn, pnn);
    load_rows(tok + stride, pn, trn, on);
    float dg[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) dg[j] = 0.f;
    F8 y[CP];
#pragma unroll
    for (int ch = 0; ch < CP; ++ch)
#pragma unroll
      for (int q = 0; q < 8; ++q) y[ch].v[q] = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int j = s / CP, ch = s % CP;
      const F8 ov = cvt8(o[s]);
#pragma unroll
      for (int q = 0; q < 8; ++q) y[ch].v[q] += g[j] * ov.v[q];
    }
#pragma unroll
    for (int ch = 0; ch < CP; ++ch) {
      const F8 tv = cvt8(tr[ch]);
      const int c = ch * 256 + hl * 8;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float r = y[ch].v[q] - tv.v[q];
        if (live && c < d) lsum += r * r;
        y[ch].v[q] = r * p.inv_tupd;   // now dL/dy
      }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int j = s / CP, ch = s % CP;
      const int c = ch * 256 + hl * 8;
      if (live && j < k && c < d) {
        const F8 ov = cvt8(o[s]);
        F8 w;
        float sdot = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          w.v[q] = g[j] * y[ch].v[q];
          sdot += y[ch].v[q] * ov.v[q];
        }
        dg[j] += sdot;
        st8(dout + (long)pos[j] * d + c, w);
      }
    }
    float sg = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
#pragma unroll
        for (int m = 16; m >= 1; m >>= 1) dg[j] += __shfl_xor(dg[j], m, 64);
        sg += g[j] * dg[j];
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (live && j < k && hl == j) p.dzsel[tok * k + j] = g[j] * (dg[j] - sg);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      g[j] = gn[j];
      pos[j] = pn[j];
      gn[j] = gnn[j];
      pn[j] = pnn[j];
    }
#pragma unroll
    for (int ch = 0; ch < CP; ++ch) tr[ch] = trn[ch];
#pragma unroll
    for (int s = 0; s < NS; ++s) o[s] = on[s];
  }
  return lsum;
}

// The pipelined form is built into the kernel for two workgroups per CU
// (large batches), where it measured faster; with one per CU it did not.
template <typename T, int OCC>
__device__ __forceinline__ void phase_combine(const KParams& p, Meta& meta) {
  float lsum;
  if constexpr (OCC == 2)
    lsum = p.k <= 2 ? (p.d <= 1024 ? combine_tokens_1chunk<T, 4>(p) : combine_tokens<T, 4>(p))
                    : (p.d <= 256 ? combine_tokens_1chunk<T, 1>(p) : combine_tokens<T, 1>(p));
  else
    lsum = p.k <= 2 ? combine_tokens<T, 4>(p) : combine_tokens<T, 1>(p);
  const float s = block_sum(lsum, meta.red);
  if (threadIdx.x == 0) p.loss_part[logical_wg()] = s;
}

// ===========================================================================
// P5: dH = (dO W2[e]^T) * G' ; dW2[e] = A_e^T dO ; router-gradient partials
// ===========================================================================
// One weight-gradient tile: g[m0.., n0..] (an [M, N] block, ld N) = A^T B
// over chunk wi.c of expert wi.e's rows, where A = rows of width M (in expert
// order, or through amap[p] / adiv) and B = rows of width N in expert order.  An unsplit tile writes (or adds to) the
// gradient and its sum of squares into norm_part[nidx]; chunk 0 of a split
// tile writes or adds likewise but leaves the sum of squares to the fix-up;
// chunks 1.. write their partial tile into part.
template <typename T, int NS, bool GA = false>
__device__ __forceinline__ void weight_grad_tile(const KParams& p, char* lds, Meta& meta, const WItem& wi,
                                                 const char* abase, const int* amap, int adiv, int M,
                                                 const char* bbase, int N, int m0, int n0, float* g, float* part,
                                                 int tpe, bool zero, int nidx, const char* aslot0 = nullptr,
                                                 long astride = 0, const char* bslot0 = nullptr, long bstride = 0) {
  const int e = wi.e, S = meta.nch[e], kc = meta.kc;
  const int r0 = S > 1 ? wi.c * kc : 0;
  const int rows = S > 1 ? min(kc, meta.wcnt[e] - r0) : meta.wcnt[e];
  const int pe = meta.off[e] + r0;
  gemm::Operand A{abase, M, amap, adiv, pe, rows, M, m0};
  gemm::Operand B{bbase, N, nullptr, 1, pe, rows, N, n0};
  // deferred weight gradients (bf16, the applying launch): the contraction
  // runs over the expert's rows of every slot, in slot order; rows [r0, r0 +
  // rows) of that concatenation, one operand piece per slot they touch
  const bool deferred = sizeof(T) == 2 && p.defer;
  const int nsl = p.slot + 1;
  if (deferred) {
    __syncthreads();   // the previous tile is done with meta.stab
    if (threadIdx.x < nsl) {
      const int s = threadIdx.x;
      const bool own = s == p.slot;
      meta.stab[0][s] = own ? meta.cnt[e] : p.slot_cnt[s * p.E + e];
      meta.stab[1][s] = own ? meta.off[e] : p.slot_off[s * p.E + e];
    }
    __syncthreads();
    zero = p.defer_zero != 0;
  }
  auto piece = [&](int s, gemm::Operand& pa, gemm::Operand& pb, int& K) {
    int pre = 0;   // the expert's rows in the slots before s
    for (int q = 0; q < s; ++q) pre += meta.stab[0][q];
    const int lo = max(r0, pre), hi = min(r0 + rows, pre + meta.stab[0][s]);
    if (lo >= hi) return false;
    const int ps = meta.stab[1][s] + lo - pre;
    pa = gemm::Operand{aslot0 + s * astride, M, nullptr, 1, ps, hi - lo, M, m0};
    pb = gemm::Operand{bslot0 + s * bstride, N, nullptr, 1, ps, hi - lo, N, n0};
    K = hi - lo;
    return true;
  };
  auto run = [&](auto&& epi, auto&& pre) {
    if constexpr (sizeof(T) == 2) {
      if (deferred) {
        gemm::tile_dma_pieces<NS, true, true, GA>(lds, nsl, piece, epi, pre);
        return;
      }
    }
    gemm::tile<T, NS, true, true, GA>(lds, A, B, rows, epi, pre);
  };
  if (wi.c > 0) {
    float* pt = part + ((long)(meta.pbase[e] + wi.c - 1) * tpe + wi.t) * (gemm::BM * gemm::BN);
    run(
        [&](int r, int c, const float (&v)[8]) {
          F8 o;
#pragma unroll
          for (int u = 0; u < 8; ++u) o.v[u] = v[u];
          st8s(pt + r * gemm::BN + c, o, p.nt_stores);
        },
        gemm::NoPre());
    return;
  }
  float sq = 0.f;
  run(
      [&](int r, int c, const float (&v)[8], const Raw8<float>& old) {
        if (m0 + r < M && n0 + c < N) {
          F8 nv = cvt8(old);
#pragma unroll
          for (int u = 0; u < 8; ++u) nv.v[u] = zero ? v[u] : nv.v[u] + v[u];
          st8s(g + (long)(m0 + r) * N + n0 + c, nv, p.nt_stores);
#pragma unroll
          for (int u = 0; u < 8; ++u) sq += nv.v[u] * nv.v[u];
        }
      },
      [&](int r, int c) {
        Raw8<float> old{};
        if (!zero && m0 + r < M && n0 + c < N) old = ldr8(g + (long)(m0 + r) * N + n0 + c);
        return old;
      });
  const float s = block_sum(sq, meta.red);
  if (S == 1 && threadIdx.x == 0) p.norm_part[nidx] = s;
}

// One element of type T at byte offset vo + so from a buffer descriptor's
// base, as fp32 (vo per lane, so uniform).
template <typename T>
__device__ __forceinline__ float ld_row_elem(gemm::rsrc_t r, int vo, int so) {
  if constexpr (sizeof(T) == 2) return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, vo, so, 0));
  else return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0));
}

// Elements of type T of 16 consecutive rows at byte offsets so + vo + u * rb
// (u = 0..15) from a buffer descriptor's base, as fp32.  The loads are one
// assembly block that ends in its own wait, so all 16 are in flight together
// (written as plain code under register pressure they were issued one at a
// time, each waited for before the next).
template <typename T>
__device__ __forceinline__ void ld_rows16(gemm::rsrc_t r, int vo, int so, int rb, float (&out)[16]) {
  uint32_t v[16];
  int off = vo;
#define MOE_LD16(OP)                                                                                           \
  asm volatile(                                                                                                \
               OP " %0, %16, %17, %18 offen\n\tv_add_u32 %16, %19, %16\n\t"                                    \
               OP " %1, %16, %17, %18 offen\n\tv_add_u32 %16, %19, %16\n\t"                                    \
               OP " %2, %16, %17, %18 offen\n\tv_add_u32 %16, %19, %16\n\t"                                    \
               OP " %3, %16, %17, %18 offen\n\tv_add_u32 %16, %19, %16\n\t"                                    \
               OP " %4, %16, %17, %18 offen\n\tv_add_u32 %16, %19, %16\n\t"                                    \
               OP " %5, %16, %17, %18 offen\n\tv_add_u32 %16, %19, %16\n\t"                                    \
               OP " %6, %16, %17, %18 offen\n\tv_add_u32 %16, %19, %16\n\t"                                    \
               OP " %7, %16, %17, %18 offen\n\tv_add_u32 %16, %19, %16\n\t"                                    \
               OP " %8, %16, %17, %18 offen\n\tv_add_u32 %16, %19, %16\n\t"                                    \
               OP " %9, %16, %17, %18 offen\n\tv_add_u32 %16, %19, %16\n\t"                                    \
               OP " %10, %16, %17, %18 offen\n\tv_add_u32 %16, %19, %16\n\t"                                   \
               OP " %11, %16, %17, %18 offen\n\tv_add_u32 %16, %19, %16\n\t"                                   \
               OP " %12, %16, %17, %18 offen\n\tv_add_u32 %16, %19, %16\n\t"                                   \
               OP " %13, %16, %17, %18 offen\n\tv_add_u32 %16, %19, %16\n\t"                                   \
               OP " %14, %16, %17, %18 offen\n\tv_add_u32 %16, %19, %16\n\t"                                   \
               OP " %15, %16, %17, %18 offen\n\t"                                                              \
               "s_waitcnt vmcnt(0)"                                                                            \
               : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),    \
                 "=&v"(v[7]), "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]), \
                 "=&v"(v[14]), "=&v"(v[15]), "+v"(off)                                                         \
               : "s"(r), "s"(so), "s"(rb)                                                                      \
               : "memory")
  if constexpr (sizeof(T) == 2) {
    MOE_LD16("buffer_load_ushort");
#pragma unroll
    for (int u = 0; u < 16; ++u) out[u] = bf16_to_f32(v[u]);
  } else {
    MOE_LD16("buffer_load_dword");
#pragma unroll
    for (int u = 0; u < 16; ++u) out[u] = __uint_as_float(v[u]);
  }
#undef MOE_LD16
}

// fp32 elements of 32 consecutive rows at byte offsets vo + u * rb (u =
// 0..31) from a buffer descriptor's base: one assembly block with its own
// wait, so all 32 loads are in flight together.
__device__ __forceinline__ void ld_rows32_f32(gemm::rsrc_t r, int vo, int rb, float (&out)[32]) {
  uint32_t v[32];
  int off = vo;
  asm volatile(
      "buffer_load_dword %0, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %1, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %2, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %3, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %4, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %5, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %6, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %7, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %8, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %9, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %10, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %11, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %12, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %13, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %14, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %15, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %16, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %17, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %18, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %19, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %20, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %21, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %22, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %23, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %24, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %25, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %26, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %27, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %28, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %29, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %30, %32, %33, 0 offen\n\tv_add_u32 %32, %34, %32\n\t"
      "buffer_load_dword %31, %32, %33, 0 offen\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),
        "=&v"(v[7]), "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]),
        "=&v"(v[14]), "=&v"(v[15]), "=&v"(v[16]), "=&v"(v[17]), "=&v"(v[18]), "=&v"(v[19]), "=&v"(v[20]),
        "=&v"(v[21]), "=&v"(v[22]), "=&v"(v[23]), "=&v"(v[24]), "=&v"(v[25]), "=&v"(v[26]), "=&v"(v[27]),
        "=&v"(v[28]), "=&v"(v[29]), "=&v"(v[30]), "=&v"(v[31]),
        "+v"(off)
      : "s"(r), "s"(rb)
      : "memory");
#pragma unroll
  for (int u = 0; u < 32; ++u) out[u] = __uint_as_float(v[u]);
}

template <typename T, int NS>
__device__ __forceinline__ void phase_bwd2(const KParams& p, char* lds, Meta& meta, bool zero_experts) {
  const int tid = threadIdx.x;
  const int G = gridDim.x, lwg = logical_wg();
  const int d = p.d, f = p.f, E = p.E, k = p.k;
  const int NTf = ceil_div(f, gemm::BN);
  const int n9 = meta.moff[E] * NTf;
  const int MT10 = ceil_div(f, gemm::BM), NT10 = ceil_div(d, gemm::BN);
  const int n10 = E * MT10 * NT10;
  const int RT = router_chunk_tokens(p.T, d, gridDim.x);
  const int RCH = ceil_div(p.T, RT), CCH = ceil_div(d, kThreads);
  const int nr = RCH * CCH;
  // G' as stored, or H (the recomputation rule) from which the epilogue forms it
  const T* gsrc = reinterpret_cast<const T*>(p.recompute ? p.act : p.gp);
  T* dh = reinterpret_cast<T*>(p.dh);
  float* gw2 = p.grads + (long)d * E + (long)E * d * f;
  const T* x = reinterpret_cast<const T*>(p.x);

  // each kind of work is dealt over the XCDs on its own, so every XCD gets the
  // same mix (the kinds differ a lot in cost)
  // (a cost-weighted deal as in dW1 + dX measured slower here at 2x1024 and
  // no faster at 32x1024)
  const DealW d10 = deal_weight_tiles(meta, E, MT10 * NT10, 0);
  const Span s9 = xcd_span(n9), sr = xcd_span_last(nr);
  // deferred weight gradients: only the applying launch has dW2 tiles
  const bool wgrad = !p.defer || p.defer_final;
  const int c10 = wgrad ? d10.count() : 0;
  const int c9 = s9.count();
  const int cr = max(0, ceil_div(sr.end - sr.begin, sr.step));
  for (int q = 0; q < c10 + c9 + cr; ++q) {
    if (q < c10) {
      // dW2[e] (f x d) = A_e^T dO_e, contraction over the expert's rows (chunk c of them)
      const WItem wi = d10.item(meta, E, q);
      const int e = wi.e, mt = wi.t / NT10, nt = wi.t % NT10;
      const int m0 = mt * gemm::BM, n0 = nt * gemm::BN;
      // under the recomputation rule act holds H: A = gelu(H) on the fragments
      if (p.recompute)
        weight_grad_tile<T, NS, true>(p, lds, meta, wi, reinterpret_cast<const char*>(p.act), nullptr, 1, f,
                                      reinterpret_cast<const char*>(p.dout), d, m0, n0, gw2 + (long)e * f * d,
                                      p.wpart2, MT10 * NT10, zero_experts, e * (MT10 * NT10) + wi.t,
                                      p.slot_act, p.stride_nf, p.slot_dout, p.stride_nd);
      else
        weight_grad_tile<T, NS, false>(p, lds, meta, wi, reinterpret_cast<const char*>(p.act), nullptr, 1, f,
                                       reinterpret_cast<const char*>(p.dout), d, m0, n0, gw2 + (long)e * f * d,
                                       p.wpart2, MT10 * NT10, zero_experts, e * (MT10 * NT10) + wi.t,
                                      p.slot_act, p.stride_nf, p.slot_dout, p.stride_nd);
      continue;
    }
    const int item = q < c10 + c9 ? n10 + s9.item(q - c10)
                                  : n10 + n9 + sr.begin + (q - c10 - c9) * sr.step;
    if (item < n10 + n9) {
      const int tI = item - n10;
      const int mg = tI / NTf, nt = tI % NTf;
      const int e = expert_of_tile(meta, E, mg);
      const int m0 = (mg - meta.moff[e]) * gemm::BM;
      const int p0 = meta.off[e] + m0;
      const int mrows = min(gemm::BM, meta.cnt[e] - m0);
      // B[k = d][n = f] = W2[e][n][k]: rows of W2[e] run along k -> direct
      gemm::Operand A{reinterpret_cast<const char*>(p.dout), d, nullptr, 1, p0, mrows, d, 0};
      gemm::Operand B{reinterpret_cast<const char*>(w2_ptr<T>(p) + (long)e * f * d), d, nullptr, 1,
                      nt * gemm::BN, min(gemm::BN, f - nt * gemm::BN), d, 0};
      const int n0 = nt * gemm::BN;
      gemm::tile<T, NS, false, false>(
          lds, A, B, d,
          [&](int r, int c, const float (&v)[8], const Raw8<T>& graw) {
            if (r < mrows && n0 + c < f) {
              F8 g8 = cvt8(graw);
              if (p.recompute) {   // graw holds H: gelu'(H) recomputed here
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                  float a, da;
                  gelu_and_grad(g8.v[u], a, da);
                  g8.v[u] = da;
                }
              }
#pragma unroll
              for (int u = 0; u < 8; ++u) g8.v[u] *= v[u];
              st8s(dh + (long)(p0 + r) * f + n0 + c, g8, p.nt_stores);
            }
          },
          [&](int r, int c) {
            Raw8<T> graw{};
            if (r < mrows && n0 + c < f) graw = ldr8(gsrc + (long)(p0 + r) * f + n0 + c);
            return graw;
          });
    } else {
      // router-gradient partial: tokens [rc*RT, +RT) x columns [cc*256, +256).
      // The chunk's dL/dz is laid out dense in LDS ([RT][EP], zero for the
      // experts a token did not select); each thread sums x[t][c] dz[t][e]
      // over the tokens in order, 16 experts at a time in registers.  The
      // selected terms are added in the same order as a sparse sum and the
      // others add zero, so no LDS read-modify-write chain is needed.
      const int ir = item - n10 - n9;
      const int rc = ir / CCH, cc = ir % CCH;
      const int t0 = rc * RT, t1 = min(p.T, t0 + RT), nt = t1 - t0;
      const int EP = (E + 15) & ~15;
      float* dzd = reinterpret_cast<float*>(lds);   // [RT][EP]
      const int c = cc * kThreads + tid;
      __syncthreads();
      for (int i = tid; i < nt * EP; i += kThreads) dzd[i] = 0.f;
      __syncthreads();
      for (int i = tid; i < nt * k; i += kThreads) dzd[(i / k) * EP + p.idx[t0 * k + i]] = p.dzsel[t0 * k + i];
      __syncthreads();
      if (c < d) {
        // x[t][c] through a buffer descriptor based at the chunk's first row
        const gemm::rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(x + (long)t0 * d), (short)0, nt * d * (int)sizeof(T), gemm::kRsrcWord3);
        const int vo = c * (int)sizeof(T), rb = d * (int)sizeof(T);
        // x values of 32 tokens requested as two blocks of 16 loads
        const int nfull = nt >> 5;
        for (int e0 = 0; e0 < E; e0 += 16) {
          float a[16];
#pragma unroll
          for (int j = 0; j < 16; ++j) a[j] = 0.f;
          for (int b = 0; b < nfull; ++b) {
            float xv[32];
            ld_rows16<T>(xr, vo, 32 * b * rb, rb, *reinterpret_cast<float(*)[16]>(&xv[0]));
            ld_rows16<T>(xr, vo, (32 * b + 16) * rb, rb, *reinterpret_cast<float(*)[16]>(&xv[16]));
#pragma unroll
            for (int u = 0; u < 32; ++u) {
              const float4* zr = reinterpret_cast<const float4*>(dzd + (32 * b + u) * EP + e0);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float4 z = zr[q];
                a[4 * q + 0] += xv[u] * z.x;
                a[4 * q + 1] += xv[u] * z.y;
                a[4 * q + 2] += xv[u] * z.z;
                a[4 * q + 3] += xv[u] * z.w;
              }
            }
          }
          for (int t = 32 * nfull; t < nt; ++t) {
            const float x1 = ld_row_elem<T>(xr, vo, t * rb);
            const float4* zr = reinterpret_cast<const float4*>(dzd + t * EP + e0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float4 z = zr[q];
              a[4 * q + 0] += x1 * z.x;
              a[4 * q + 1] += x1 * z.y;
              a[4 * q + 2] += x1 * z.z;
              a[4 * q + 3] += x1 * z.w;
            }
          }
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (e0 + j < E) p.rpart[((long)rc * E + e0 + j) * d + c] = a[j];
        }
      }
    }
  }
}

// ===========================================================================
// P6: dW1[e] = X_e^T dH ; dXs = dH W1[e]^T ; router gradient reduction
// ===========================================================================
template <typename T, int NS>
__device__ __forceinline__ void phase_bwd1(const KParams& p, char* lds, Meta& meta, bool zero_router, bool zero_experts,
                                           bool want_dx, bool fix_dw2) {
  const int tid = threadIdx.x;
  const int G = gridDim.x, lwg = logical_wg();
  const int d = p.d, f = p.f, E = p.E;
  const int MT11 = ceil_div(d, gemm::BM), NT11 = ceil_div(f, gemm::BN);
  const int n11 = E * MT11 * NT11;
  const int NTd = ceil_div(d, gemm::BN);
  const int n12 = want_dx ? meta.moff[E] * NTd : 0;
  const int nrr = ceil_div(d * E, kThreads);
  const int n10 = E * ceil_div(f, gemm::BM) * ceil_div(d, gemm::BN);
  const int RCH = ceil_div(p.T, router_chunk_tokens(p.T, d, gridDim.x));
  float* gw1 = p.grads + (long)d * E;
  T* dxs = reinterpret_cast<T*>(p.dxs);

  DealW d11 = deal_weight_tiles(meta, E, MT11 * NT11, 1);
  // deferred weight gradients: only the applying launch has dW1 tiles
  const bool wgrad = !p.defer || p.defer_final;
  Span s12 = xcd_span(n12);
  const Span srr = xcd_span_last(nrr);
  // dW1 tiles: k-tiles over the mean rows per expert; dX tiles: over f.  Built
  // into the kernel for two workgroups per CU only (large batches), where it
  // measured faster; in the other kernel its code alone cost more than it saved.
  if constexpr (NS == 2)
    if (!d11.snake && wgrad) cost_deal(n11, ceil_div(meta.wtot, 64 * E) + 6, n12, ceil_div(f, 64) + 3, d11.sp, s12);
  // fix-ups of the dW2 tiles whose contraction was split in the previous phase
  const int tpe10 = ceil_div(f, gemm::BM) * ceil_div(d, gemm::BN);
  const int nfx = fix_dw2 ? meta.nsplit * tpe10 : 0;
  const Span sfx = xcd_span(nfx);
  const int c11 = wgrad ? d11.count() : 0;
  const int c12 = s12.count();
  const int crr = max(0, ceil_div(srr.end - srr.begin, srr.step));
  const int cfx = max(0, ceil_div(sfx.end - sfx.begin, sfx.step));
  for (int q = 0; q < c11 + c12 + crr + cfx; ++q) {
    if (q < c11) {
      // dW1[e] (d x f) = X_e^T dH_e over chunk c of the expert's rows; bf16: the
      // token rows gathered in route_order; fp32: x through perm
      const WItem wi = d11.item(meta, E, q);
      const int e = wi.e, mt = wi.t / NT11, nt = wi.t % NT11;
      const int m0 = mt * gemm::BM, n0 = nt * gemm::BN;
      weight_grad_tile<T, NS>(p, lds, meta, wi,
                              sizeof(T) == 2 ? reinterpret_cast<const char*>(p.xs) : reinterpret_cast<const char*>(p.x),
                              sizeof(T) == 2 ? nullptr : p.perm, sizeof(T) == 2 ? 1 : p.k, d,
                              reinterpret_cast<const char*>(p.dh), f, m0, n0, gw1 + (long)e * d * f, p.wpart1,
                              MT11 * NT11, zero_experts, n10 + e * (MT11 * NT11) + wi.t, p.slot_xs, p.stride_nd,
                              p.slot_dh, p.stride_nf);
      continue;
    }
    if (q >= c11 + c12 + crr) {
      const int u = sfx.begin + (q - c11 - c12 - crr) * sfx.step;
      const int e = meta.splitlist[u / tpe10], t = u % tpe10;
      const float sq = fix_split_tile(meta, p.grads + (long)d * E + (long)E * d * f + (long)e * f * d, p.wpart2, e, t,
                                      f, d, ceil_div(d, gemm::BN));
      const float s = block_sum(sq, meta.red);
      if (tid == 0) p.norm_part[e * tpe10 + t] = s;
      continue;
    }
    const int item = q < c11 + c12 ? n11 + s12.item(q - c11)
                                   : n11 + n12 + srr.begin + (q - c11 - c12) * srr.step;
    if (item < n11 + n12) {
      const int tI = item - n11;
      const int mg = tI / NTd, nt = tI % NTd;
      const int e = expert_of_tile(meta, E, mg);
      const int m0 = (mg - meta.moff[e]) * gemm::BM;
      const int p0 = meta.off[e] + m0;
      const int mrows = min(gemm::BM, meta.cnt[e] - m0);
      // B[k = f][n = d] = W1[e][n][k]: rows of W1[e] run along k -> direct
      gemm::Operand A{reinterpret_cast<const char*>(p.dh), f, nullptr, 1, p0, mrows, f, 0};
      gemm::Operand B{reinterpret_cast<const char*>(w1_ptr<T>(p) + (long)e * d * f), f, nullptr, 1,
                      nt * gemm::BN, min(gemm::BN, d - nt * gemm::BN), f, 0};
      const int n0 = nt * gemm::BN;
      gemm::tile<T, NS, false, false>(
          lds, A, B, f,
          [&](int r, int c, const float (&v)[8], int slot) {
            if (r < mrows && n0 + c < d) {
              F8 o;
#pragma unroll
              for (int u = 0; u < 8; ++u) o.v[u] = v[u];
              st8s(dxs + (long)slot * d + n0 + c, o, p.nt_stores);
            }
          },
          [&](int r, int c) { return (r < mrows && n0 + c < d) ? p.perm[p0 + r] : 0; });
    } else {
      // dW_r[c][e] = sum over token chunks (ascending) of the partials
      // one (expert, column) pair per thread, columns consecutive across the
      // threads so every chunk's partials are read in 1 KB pieces; the chunk
      // partials are added in ascending chunk order, 32 loads in flight
      const int ir = item - n11 - n12;
      const int o = ir * kThreads + tid;
      float sq = 0.f;
      if (o < d * E) {
        const int e = o / d, c = o % d;
        const float* src = p.rpart + (long)e * d + c;
        const long stride = (long)E * d;
        float s = 0.f;
        int r = 0;
        for (; r + 32 <= RCH; r += 32) {
          // a descriptor based at chunk r's partials: 32 chunk rows of E * d floats
          const gemm::rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
              (void*)(p.rpart + (long)r * stride), (short)0, (int)(32 * stride * 4), gemm::kRsrcWord3);
          float v[32];
          ld_rows32_f32(rr, o * 4, (int)(stride * 4), v);
#pragma unroll
          for (int u = 0; u < 32; ++u) s += v[u];
        }
        for (; r + 8 <= RCH; r += 8) {
          float v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = src[(r + u) * stride];
#pragma unroll
          for (int u = 0; u < 8; ++u) s += v[u];
        }
        for (; r < RCH; ++r) s += src[r * stride];
        const int gi = c * E + e;   // W_r is [d, E]
        const float nv = zero_router ? s : p.grads[gi] + s;
        p.grads[gi] = nv;
        sq = nv * nv;
      }
      const float s = block_sum(sq, meta.red);
      if (tid == 0) p.norm_part[n10 + n11 + ir] = s;
    }
  }
}

// ===========================================================================
// P7: dx row sums; global norm; clip + AdamW (+ bf16 weight copy)
// ===========================================================================
// dx of each token = router part sum_j dz_j W_r[:, e_j] + the token's k slot
// rows of dXs, summed in slot order.  wrt is W_r^T, in LDS when it fits (each
// token reads k rows of it).  One token per half-wave as in the
// combine phase: lane h owns columns 8h.. of each 256-column chunk, CP chunks
// are loaded at once, and the next token's dz / experts are loaded one token
// ahead.
template <typename T, int CP>
__device__ __forceinline__ void dx_tokens(const KParams& p, const float* wrt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, hl = lane & 31;
  const int G = gridDim.x, lwg = logical_wg();
  const int d = p.d, k = p.k;
  const T* dxs = reinterpret_cast<const T*>(p.dxs);
  const int stride = G * kWaves * 2;
  constexpr int NS = CP * kMaxTopK > 8 ? 8 : CP * kMaxTopK;
  float dz[kMaxTopK], dzn[kMaxTopK];
  int ev[kMaxTopK], evn[kMaxTopK];
  auto load_idx = [&](int tok, float (&zz)[kMaxTopK], int (&ee)[kMaxTopK]) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      zz[j] = 0.f;
      ee[j] = 0;
      if (j < k && tok < p.T) {
        zz[j] = p.dzsel[tok * k + j];
        ee[j] = p.idx[tok * k + j];
      }
    }
  };
  int base = wave * 2 * G + lwg;   // token of half-wave 0; half-wave 1 takes base + G
  load_idx(base + half * G, dz, ev);
  for (; base < p.T; base += stride) {
    const int tok = base + half * G;
    const bool live = tok < p.T;
    load_idx(tok + stride, dzn, evn);
    for (int c0 = 0; c0 < d; c0 += 256 * CP) {
      Raw8<float> w[NS];
      Raw8<T> v[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int j = s / CP, ch = s % CP;
        const int c = c0 + ch * 256 + hl * 8;
        w[s] = Raw8<float>{};
        v[s] = Raw8<T>{};
        if (live && j < k && c < d) {
          w[s] = ldr8(wrt + (long)ev[j] * d + c);
          v[s] = ldr8(dxs + ((long)tok * k + j) * d + c);
        }
      }
      F8 acc[CP];
#pragma unroll
      for (int ch = 0; ch < CP; ++ch)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[ch].v[q] = 0.f;
      // router part first, then the slot rows, each in slot order
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int j = s / CP, ch = s % CP;
        const F8 wf = cvt8(w[s]);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[ch].v[q] += dz[j] * wf.v[q];
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int j = s / CP, ch = s % CP;
        if (j < k) {
          const F8 vf = cvt8(v[s]);
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[ch].v[q] += vf.v[q];
        }
      }
#pragma unroll
      for (int ch = 0; ch < CP; ++ch) {
        const int c = c0 + ch * 256 + hl * 8;
        if (live && c < d) st8(p.dx + (long)tok * d + c, acc[ch]);
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      dz[j] = dzn[j];
      ev[j] = evn[j];
    }
  }
}

template <typename T, int OCC>
__device__ __forceinline__ void phase_final(const KParams& p, char* smem, Meta& meta, bool restart_loss, bool apply_r,
                                            bool apply_e, bool want_dx) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = gridDim.x, lwg = logical_wg();
  const int d = p.d, f = p.f, E = p.E, k = p.k;

  if (want_dx && !(p.flags & 0x200000u)) {
    // the router part reads a row of W_r^T per slot: from LDS when W_r^T fits
    // the scratch and the workgroup has at least 32 tokens (staging costs a
    // workgroup about as much as 16 tokens' reads from L2: measured slower at
    // 4 and 16 tokens per workgroup, faster at 64), else from L2
    constexpr int kScratch = scratch_bytes(OCC);
    const bool staged = (long)E * d * 4 <= kScratch && ((E * d) & 3) == 0 && p.T >= 32 * G;
    if (staged) {
      float4* dst = reinterpret_cast<float4*>(smem);
      const float4* src = reinterpret_cast<const float4*>(p.wrt);
      for (int i = tid; i < E * d / 4; i += kThreads) dst[i] = src[i];
      __syncthreads();
    }
    // (separate calls, so the staged reads compile to LDS reads)
    if (staged) p.k <= 2 ? dx_tokens<T, 4>(p, reinterpret_cast<const float*>(smem))
                         : dx_tokens<T, 1>(p, reinterpret_cast<const float*>(smem));
    else p.k <= 2 ? dx_tokens<T, 4>(p, p.wrt) : dx_tokens<T, 1>(p, p.wrt);
    __syncthreads();   // the scratch is reused below
  }

  // loss of this launch, summed over workgroups in index order
  if (lwg == 0 && p.stats) {
    float* red = reinterpret_cast<float*>(smem);
    float s = 0.f;
    for (int w = tid; w < G; w += kThreads) s += p.loss_part[w];
    red[tid] = s;
    __syncthreads();
    if (tid == 0) {
      float tot = 0.f;
      for (int i = 0; i < kThreads; ++i) tot += red[i];
      tot *= 0.5f * p.inv_tupd;
      p.stats[0] = restart_loss ? tot : p.stats[0] + tot;
    }
    __syncthreads();
  }
  if (!apply_r && !apply_e) return;

  // global norm from the per-tile partials of the applied groups (the expert
  // tiles first, then the router items), fixed order (same in every workgroup)
  const int n10 = E * ceil_div(f, gemm::BM) * ceil_div(d, gemm::BN);
  const int n11 = E * ceil_div(d, gemm::BM) * ceil_div(f, gemm::BN);
  const int nrr = ceil_div(d * E, kThreads);
  const int q0 = apply_e ? 0 : n10 + n11, q1 = apply_r ? n10 + n11 + nrr : n10 + n11;
  float* red = reinterpret_cast<float*>(smem);
  {
    float s = 0.f;
    for (int i = q0 + tid; i < q1; i += kThreads) s += p.norm_part[i];
    __syncthreads();
    red[tid] = s;
    __syncthreads();
    if (tid == 0) {
      float tot = 0.f;
      for (int i = 0; i < kThreads; ++i) tot += red[i];
      red[kThreads] = tot;
    }
    __syncthreads();
  }
  const float norm = sqrtf(red[kThreads]);
  const float c = (p.clip > 0.f) ? fminf(1.f, p.clip / (norm + 1e-6f)) : 1.f;
  if (lwg == 0 && tid == 0 && p.stats) {
    p.stats[1] = norm;
    p.stats[2] = c;
  }

  // clip + AdamW over the flat parameter vector, 4 parameters per thread-step
  const long P = (long)d * E + 2L * E * d * f;
  const long P4 = P / 4;
  const long nr4 = (long)d * E / 4;
  const float b1 = p.beta1, b2 = p.beta2, omb1 = p.omb1, omb2 = p.omb2, lr = p.lr, eps = p.eps, wd = p.wd;
  // W_r is the float4 range [0, nr4), W1 | W2 the rest; each group has its own
  // bias correction, and only the applied groups are updated
  const long lo4 = apply_r ? 0 : nr4, hi4 = apply_e ? P4 : nr4;
  float4* P_ = reinterpret_cast<float4*>(p.params);
  const float4* G_ = reinterpret_cast<const float4*>(p.grads);
  float4* M_ = reinterpret_cast<float4*>(p.m);
  float4* V_ = reinterpret_cast<float4*>(p.v);
  // every parameter, gradient and moment is touched once per update: stream them
  // with non-temporal loads and stores so they do not evict reused data
  typedef float nt4 __attribute__((ext_vector_type(4)));
  auto adamw4 = [&](long i, float4& w, const float4& g, float4& m, float4& v) {
    const int grp = i < nr4 ? 0 : 1;
    const float ib1 = p.inv_bc1[grp], isb2 = p.inv_sqrt_bc2[grp];
    float* wv = &w.x;
    const float* gv = &g.x;
    float* mv = &m.x;
    float* vv = &v.x;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float gc = c * gv[q];
      mv[q] = b1 * mv[q] + omb1 * gc;
      vv[q] = b2 * vv[q] + omb2 * gc * gc;
      const float upd = (mv[q] * ib1) / (sqrtf(vv[q]) * isb2 + eps) + wd * wv[q];
      wv[q] = wv[q] - lr * upd;
    }
  };
  auto store4 = [&](long i, const float4& w, const float4& m, const float4& v) {
    __builtin_nontemporal_store(nt4{w.x, w.y, w.z, w.w}, reinterpret_cast<nt4*>(P_ + i));
    __builtin_nontemporal_store(nt4{m.x, m.y, m.z, m.w}, reinterpret_cast<nt4*>(M_ + i));
    __builtin_nontemporal_store(nt4{v.x, v.y, v.z, v.w}, reinterpret_cast<nt4*>(V_ + i));
    if (p.shadow && i >= nr4) {
      uint2 s;
      s.x = pack_bf16x2(w.x, w.y);
      s.y = pack_bf16x2(w.z, w.w);
      reinterpret_cast<uint2*>(p.shadow)[i - nr4] = s;
    }
  };
  // loads in flight per thread: four of each array with a SIMD's full register
  // file, two with half of it (twice the workgroups keep as many in flight)
  constexpr int U = OCC == 1 ? 4 : 2;
  const long stride = (long)G * kThreads;
  long i = lo4 + (long)lwg * kThreads + tid;
  for (; i + (U - 1) * stride < hi4; i += U * stride) {
    float4 w[U], g[U], m[U], v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      nt4 a0 = __builtin_nontemporal_load(reinterpret_cast<const nt4*>(P_ + i + u * stride));
      nt4 a1 = __builtin_nontemporal_load(reinterpret_cast<const nt4*>(G_ + i + u * stride));
      nt4 a2 = __builtin_nontemporal_load(reinterpret_cast<const nt4*>(M_ + i + u * stride));
      nt4 a3 = __builtin_nontemporal_load(reinterpret_cast<const nt4*>(V_ + i + u * stride));
      w[u] = make_float4(a0.x, a0.y, a0.z, a0.w);
      g[u] = make_float4(a1.x, a1.y, a1.z, a1.w);
      m[u] = make_float4(a2.x, a2.y, a2.z, a2.w);
      v[u] = make_float4(a3.x, a3.y, a3.z, a3.w);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      adamw4(i + u * stride, w[u], g[u], m[u], v[u]);
      store4(i + u * stride, w[u], m[u], v[u]);
    }
  }
  for (; i < hi4; i += stride) {
    float4 w = P_[i], g = G_[i], m = M_[i], v = V_[i];
    adamw4(i, w, g, m, v);
    store4(i, w, m, v);
  }
}

// ===========================================================================
// The persistent kernel: one launch per update (or microbatch)
// ===========================================================================
// The launch's KParams, read from the kernel-argument segment.  The pointer
// passes through an empty asm statement at each call, so the compiler cannot
// prove two calls equal: each phase loads the fields it uses (scalar loads
// from the constant cache) instead of keeping all of the structure in scalar
// registers for the whole launch, which the scalar register file cannot hold.
__device__ __forceinline__ const KParams& kernel_args() {
  using ArgPtr = const __attribute__((address_space(4))) KParams*;
  ArgPtr q = (ArgPtr)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(q));
  return *(const KParams*)q;
}

template <typename T, int OCC>
__global__ void __launch_bounds__(kThreads, OCC) moe_step_kernel(KParams args) {
  (void)args;   // read through kernel_args(), phase by phase
  constexpr int NS = dma_stages(OCC);
  extern __shared__ __align__(16) char smem_raw[];
  Meta& meta = *reinterpret_cast<Meta*>(smem_raw);
  char* work = smem_raw + kMetaBytes;   // LDS after the routing metadata
  // the host has expanded the whole-update bits into the per-group ones
  const unsigned flags = kernel_args().flags;
  const bool zero_r = (flags & 0x10u) != 0u, zero_e = (flags & 0x20u) != 0u;
  const bool apply_r = (flags & 0x40u) != 0u, apply_e = (flags & 0x80u) != 0u;

  int hk = 0;   // barriers passed in this launch (the first one learns the XCD membership)
#define MOE_SYNC(ph)                                                                    \
  do {                                                                                  \
    const KParams& pb = kernel_args();                                                  \
    trace_mark(pb, ph, 1);                                                              \
    if (!grid_barrier(pb.ctrl, pb.epoch * 8u + (ph) + 1u, &meta.bar, hk++)) return;     \
    trace_mark(pb, ph, 2);                                                              \
  } while (0)

  // A launch enqueued after one that gave up (before moe_step_status reset the
  // abort word) writes nothing.
  if (threadIdx.x == 0)
    meta.bar.flag = __hip_atomic_load(kernel_args().ctrl.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (meta.bar.flag != 0u) return;
  if ((flags & 0x40000u) && blockIdx.x == gridDim.x - 1) {
    // failure-path test: this workgroup waits for a word nothing sets, gives
    // up, and never arrives at the first barrier
    if (threadIdx.x == 0) (void)wait_for(kernel_args().ctrl, kernel_args().ctrl.never, 1u);
    return;
  }
  const unsigned skip = flags >> 8;
  trace_mark(kernel_args(), 0, 0);
  if (!(skip & 1u)) phase_route<T, OCC>(kernel_args(), work, meta);
  MOE_SYNC(0);
  trace_mark(kernel_args(), 1, 0);
  phase_order<T>(kernel_args(), work, meta, (skip & 2u) != 0u);   // the offsets are always rebuilt
  MOE_SYNC(1);
  trace_mark(kernel_args(), 2, 0);
  const bool ready12 = (flags & 0x10000u) != 0u;
  if (!(skip & 4u)) phase_ffn1<T, NS>(kernel_args(), work, meta, ready12);
  if (ready12) {   // readiness counters instead of a grid barrier
    trace_mark(kernel_args(), 2, 1);
    trace_mark(kernel_args(), 2, 2);
  } else {
    MOE_SYNC(2);
  }
  trace_mark(kernel_args(), 3, 0);
  if (!(skip & 8u) && !phase_ffn2<T, NS>(kernel_args(), work, meta, ready12 && !(skip & 4u))) return;
  MOE_SYNC(3);
  trace_mark(kernel_args(), 4, 0);
  if (!(skip & 16u)) phase_combine<T, OCC>(kernel_args(), meta);
  MOE_SYNC(4);
  trace_mark(kernel_args(), 5, 0);
  if (!(skip & 32u)) phase_bwd2<T, NS>(kernel_args(), work, meta, zero_e);
  MOE_SYNC(5);
  trace_mark(kernel_args(), 6, 0);
  const bool want_dx = kernel_args().dx != nullptr;
  if (!(skip & 64u)) phase_bwd1<T, NS>(kernel_args(), work, meta, zero_r, zero_e, want_dx, !(skip & 32u));
  MOE_SYNC(6);
  if (meta.nsplit > 0 && !(skip & 64u)) {
    // complete the dW1 tiles whose contraction was split, so the global norm
    // below sees whole gradients; a grid barrier separates the two
    const KParams& p = kernel_args();
    const int d = p.d, f = p.f, E = p.E;
    const int tpe = ceil_div(d, gemm::BM) * ceil_div(f, gemm::BN);
    const int n10 = E * ceil_div(f, gemm::BM) * ceil_div(d, gemm::BN);
    const Span sp = xcd_span(meta.nsplit * tpe);
    for (int u = sp.begin; u < sp.end; u += sp.step) {
      const int e = meta.splitlist[u / tpe], t = u % tpe;
      const float sq = fix_split_tile(meta, p.grads + (long)d * E + (long)e * d * f, p.wpart1, e, t, d, f,
                                      ceil_div(f, gemm::BN));
      const float s = block_sum(sq, meta.red);
      if (threadIdx.x == 0) p.norm_part[n10 + e * tpe + t] = s;
    }
    if (!grid_barrier(p.ctrl, p.epoch * 8u + 8u, &meta.bar, hk++)) return;
  }
  trace_mark(kernel_args(), 7, 0);
  if (!(skip & 128u)) phase_final<T, OCC>(kernel_args(), work, meta, zero_r || zero_e, apply_r, apply_e, want_dx);
  __syncthreads();
  trace_mark(kernel_args(), 7, 1);
  trace_mark(kernel_args(), 7, 2);
#undef MOE_SYNC
}

}  // namespace moe
