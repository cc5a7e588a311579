// Host side of the C ABI declared in include/moe_step.h: validation, the device
// arena, and one launch of the persistent kernel per update (ordinary by
// default, cooperative on request).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "../../include/moe_step.h"
#include "phases.h"

namespace {

thread_local char g_create_error[512] = "no error";

void set_err(char* buf, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, 512, fmt, ap);
  va_end(ap);
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int cdiv(int a, int b) { return (a + b - 1) / b; }

int check_config(const moe_step_config* c, char* err) {
  if (!c) { set_err(err, "config is NULL"); return MOE_ERR_ARG; }
  if (c->struct_size != sizeof(moe_step_config)) {
    set_err(err, "config.struct_size %u != %zu", c->struct_size, sizeof(moe_step_config));
    return MOE_ERR_ARG;
  }
  if (c->abi_version != MOE_STEP_ABI_VERSION) {
    set_err(err, "config.abi_version %u != %u", c->abi_version, MOE_STEP_ABI_VERSION);
    return MOE_ERR_ARG;
  }
  if (c->d_model <= 0 || c->d_ff <= 0 || c->n_experts <= 0 || c->top_k <= 0 || c->max_tokens <= 0) {
    set_err(err, "dimensions must be positive (d=%d f=%d E=%d k=%d max_tokens=%d)", c->d_model, c->d_ff,
            c->n_experts, c->top_k, c->max_tokens);
    return MOE_ERR_ARG;
  }
  if (c->dtype != MOE_DTYPE_F32 && c->dtype != MOE_DTYPE_BF16) {
    set_err(err, "unknown dtype %d", c->dtype);
    return MOE_ERR_ARG;
  }
  if (!(c->lr >= 0.0) || !(c->beta1 >= 0.0 && c->beta1 < 1.0) || !(c->beta2 >= 0.0 && c->beta2 < 1.0) ||
      !(c->adam_eps >= 0.0) || !(c->weight_decay >= 0.0) || std::isnan(c->clip_norm)) {
    set_err(err, "optimizer hyper-parameters out of range");
    return MOE_ERR_ARG;
  }
  if (c->memory_rules & ~(MOE_MEM_RECOMPUTE | MOE_MEM_GUARDS)) {
    set_err(err, "unknown memory rules 0x%x", c->memory_rules);
    return MOE_ERR_ARG;
  }
  if (c->max_microbatches < 0 || c->max_microbatches > moe::kMaxSlots) {
    set_err(err, "max_microbatches must be in [0, %d]", moe::kMaxSlots);
    return MOE_ERR_ARG;
  }
  if (c->max_microbatches > 1 && (c->dtype != MOE_DTYPE_BF16 || (c->memory_rules & MOE_MEM_RECOMPUTE))) {
    set_err(err, "deferred weight gradients (max_microbatches > 1) need a bf16 handle without MOE_MEM_RECOMPUTE");
    return MOE_ERR_ARG;
  }
  if ((long long)c->max_microbatches * c->max_tokens * c->top_k >= (1LL << 30)) {
    set_err(err, "max_microbatches * max_tokens * top_k must stay below 2^30");
    return MOE_ERR_SHAPE;
  }
  if (c->wg_per_cu < 0 || c->wg_per_cu > 2) {
    set_err(err, "wg_per_cu must be 0, 1 or 2");
    return MOE_ERR_ARG;
  }
  if (c->top_k > c->n_experts) {
    set_err(err, "top_k %d > n_experts %d", c->top_k, c->n_experts);
    return MOE_ERR_ARG;
  }
  if (c->d_model % 8 || c->d_ff % 8) {
    set_err(err, "d_model and d_ff must be multiples of 8 (got %d, %d)", c->d_model, c->d_ff);
    return MOE_ERR_SHAPE;
  }
  if (c->n_experts > moe::kMaxExperts) {
    set_err(err, "n_experts %d > %d", c->n_experts, moe::kMaxExperts);
    return MOE_ERR_SHAPE;
  }
  if (c->top_k > moe::kMaxTopK) {
    set_err(err, "top_k %d > %d", c->top_k, moe::kMaxTopK);
    return MOE_ERR_SHAPE;
  }
  if (c->max_tokens > (1 << 24)) {
    set_err(err, "max_tokens %d > 2^24", c->max_tokens);
    return MOE_ERR_SHAPE;
  }
  const long long P = (long long)c->d_model * c->n_experts + 2LL * c->n_experts * c->d_model * c->d_ff;
  if (P >= (1LL << 31) * 4LL) {
    set_err(err, "too many parameters");
    return MOE_ERR_SHAPE;
  }
  if ((long long)c->max_tokens * c->top_k * (long long)(c->d_model > c->d_ff ? c->d_model : c->d_ff) >=
      (1LL << 40)) {
    set_err(err, "activation arena too large");
    return MOE_ERR_SHAPE;
  }
  return MOE_OK;
}

}  // namespace

// Barrier words of a grid of G workgroups: generation, status, abort, an unused
// word, one arrival slot per workgroup, then the per-XCD words; 128 bytes each.
static size_t ctrl_words(int G) { return (size_t)(G + 4) * 32 + moe::kXcdWords; }

// Routed rows (max_tokens * top_k) from which a bf16 handle runs two workgroups
// per compute unit by default.
// Measured on the 768/1536/16-expert layer (C++ driver, one update per launch):
// one per CU wins at 1024 and 2048 rows, two per CU from 4096 (2x1024: 0.444
// against 0.451 ms; 4x1024: 0.52 against 0.59 ms).
constexpr long kTwoPerCuRows = 4096;

// Routed rows of a launch (n_tokens * top_k) from which the product outputs are
// written with non-temporal stores.  Measured on the same layer (C++ driver,
// one box): plain stores win at 2x1024 (0.421 against 0.490 ms) and tie on the
// Zipf workload's 8192-token microbatches; non-temporal ones win at 32x1024
// (1.723 against 1.756 ms).  With deferred weight gradients the outputs go to
// a fresh slot every launch, and at the Zipf microbatches (16,384 rows)
// non-temporal stores win (7.59 against 7.74 ms per update; without deferral
// they lose there, 8.90 against 8.82 ms, same box).
constexpr long kNonTemporalRows = 32768;
constexpr long kNonTemporalRowsDeferred = 16384;

struct moe_step {
  moe_step_config cfg;
  int grid = 0;
  int cus = 0;
  int occ = 1;                  // workgroups per compute unit the kernel is built for
  const void* kern = nullptr;   // that kernel
  int smem = 0;                 // its dynamic LDS bytes per workgroup
  char* arena = nullptr;
  size_t arena_bytes = 0;
  hipStream_t last_stream = nullptr;
  bool launched = false;
  int last_full_tokens = -1;   // n_tokens of the last launch that ran every phase
  unsigned epoch = 0;          // launches so far (barrier targets are unique per launch)
  char err[512] = "no error";
  // arena sub-buffers
  int* idx;
  float* gate;
  float* dzsel;
  int* hist;
  int* ready;
  int nrb = 0;
  int* perm;
  int* inv;
  void* act;
  void* gp;
  float* out;
  void* dout;
  void* dh;
  void* dxs;
  float* wrt;
  float* rpart;
  float* loss_part;
  float* norm_part;
  uint16_t* shadow;
  void* xs;
  float* wpart2;
  float* wpart1;
  int wpart_sets = 0;
  unsigned* ctrl;
  // guard zones of a MOE_MEM_GUARDS handle: the arena offset of each zone and
  // the sub-buffer it follows
  struct Guard {
    size_t off, len;
    const char* after;
  };
  Guard guards[32];   // plan_arena takes at most 26 sub-buffers
  int n_guards = 0;
  // deferred weight gradients (cfg.max_microbatches > 1): per-slot arrays and
  // the slot of the last launch (-1: the experts were applied, or none yet)
  char* slot_act = nullptr;
  char* slot_dout = nullptr;
  char* slot_xs = nullptr;
  char* slot_dh = nullptr;
  long stride_nf = 0, stride_nd = 0;
  int* slot_cnt = nullptr;
  int* slot_off = nullptr;
  int defer_slot = -1;
  bool defer_zero = false;
};

// Chooses the kernel (element type, workgroups per compute unit), sets its LDS
// attribute and sizes the persistent grid to what the device holds at once.
// No allocation.
static int select_kernel(const moe_step_config& c, int cus, moe_step& h, char* err) {
  // Two workgroups per compute unit pay off once the expert products have
  // many tiles (each workgroup's waits are covered by the other's matrix
  // work); small batches keep one, with the deeper pipeline and fewer
  // workgroups at every grid barrier.  The fp32 kernel is built for one.
  int want = c.wg_per_cu;
  if (want == 0) want = (c.dtype == MOE_DTYPE_BF16 && (long)c.max_tokens * c.top_k >= kTwoPerCuRows) ? 2 : 1;
  const int occ = (c.dtype == MOE_DTYPE_BF16 && want == 2) ? 2 : 1;
  const void* kern = c.dtype == MOE_DTYPE_F32 ? reinterpret_cast<const void*>(&moe::moe_step_kernel<float, 1>)
                     : occ == 2               ? reinterpret_cast<const void*>(&moe::moe_step_kernel<uint16_t, 2>)
                                              : reinterpret_cast<const void*>(&moe::moe_step_kernel<uint16_t, 1>);
  const int smem = moe::smem_bytes(occ);
  hipError_t he = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (he != hipSuccess) {
    set_err(err, "hipFuncSetAttribute(shared memory %d): %s", smem, hipGetErrorString(he));
    return MOE_ERR_HIP;
  }
  int per_cu = 0;
  he = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, moe::kThreads, smem);
  if (he != hipSuccess || per_cu < 1) {
    set_err(err, "occupancy query failed or zero (%s, %d)", hipGetErrorString(he), per_cu);
    return MOE_ERR_HIP;
  }
  h.cus = cus;
  h.grid = cus * (occ < per_cu ? occ : per_cu);
  h.occ = occ;
  h.kern = kern;
  h.smem = smem;
  return MOE_OK;
}

// Lays out the arena of h (h.cfg and h.grid set) and returns its size in
// bytes; with a base address, also points h's sub-buffers into it.  The
// barrier words (ctrl_words of them) come first.
static size_t plan_arena(moe_step& h, char* base, size_t ctrl_words) {
  const moe_step_config& c = h.cfg;
  const int d = c.d_model, f = c.d_ff, E = c.n_experts, k = c.top_k;
  const size_t Tm = (size_t)c.max_tokens, N = Tm * k;
  const size_t es = c.dtype == MOE_DTYPE_BF16 ? 2 : 4;
  const int n10 = E * cdiv(f, moe::gemm::BM) * cdiv(d, moe::gemm::BN);
  const int n11 = E * cdiv(d, moe::gemm::BM) * cdiv(f, moe::gemm::BN);
  const int nrr = cdiv(d * E, moe::kThreads);
  // router-gradient partial chunks: the most any token count up to max_tokens
  // uses.  The chunk is 128, 64 or 32 tokens over three ranges of the token
  // count, and within each range the chunk count grows with it, so the
  // largest token count of each range (clipped to max_tokens) gives the bound.
  size_t rch = 1;
  {
    const int m = cdiv(h.grid, cdiv(d, moe::kThreads));
    const int cand[3] = {c.max_tokens, std::min(c.max_tokens, 128 * (m - 1)), std::min(c.max_tokens, 64 * (m - 1))};
    for (int t : cand)
      if (t >= 1) rch = std::max(rch, (size_t)cdiv(t, moe::router_chunk_tokens(t, d, h.grid)));
  }
  // MOE_MEM_GUARDS: a zone after every sub-buffer, zero like the rest of the
  // arena at create, that no kernel may write.  At least 1 MiB, and at least
  // 128 rows of the widest fp32 row, so that a whole tile written past a
  // buffer's end stays inside the zone.
  const bool guarded = (c.memory_rules & MOE_MEM_GUARDS) != 0u;
  const size_t kGuardBytes = std::max((size_t)1 << 20, (size_t)moe::gemm::BM * std::max(d, f) * 4);
  constexpr int kMaxGuards = (int)(sizeof(h.guards) / sizeof(h.guards[0]));
  h.n_guards = 0;
  size_t off = 0;
  auto take = [&](const char* name, size_t bytes) {
    size_t o = off;
    off = align_up(off + (bytes ? bytes : 1), 256);
    if (guarded && h.n_guards < kMaxGuards) {   // from the byte after the buffer on, its padding included
      off += kGuardBytes;
      h.guards[h.n_guards++] = {o + bytes, off - (o + bytes), name};
    }
    return o;
  };
  const size_t o_ctrl = take("ctrl", ctrl_words * sizeof(unsigned));
  const size_t o_idx = take("idx", N * 4), o_gate = take("gate", N * 4), o_dz = take("dz", N * 4);
  const size_t o_hist = take("hist", (size_t)h.grid * E * 4);
  const size_t o_perm = take("perm", N * 4), o_inv = take("inv", N * 4);
  // Stored activations share memory where their lifetimes (phases between the
  // grid barriers) do not overlap:
  //   O  [N, d] fp32: written by GEMM 2, last read by the combine;
  //   dH [N, f]:      written by the dH tiles after the combine's barrier;
  //   A  [N, f]:      written by GEMM 1, last read by the dW2 tiles;
  //   dXs [N, d]:     written by the dX tiles after that phase's barrier.
  // With deferred weight gradients A, dH, dO and X_e live in per-slot arrays
  // until the applying launch, so O and dXs get buffers of their own.
  const bool defer = c.max_microbatches > 1;
  const size_t M = defer ? (size_t)c.max_microbatches : 0;
  const size_t o_out_dh = take("out_dh", defer ? N * d * 4 : std::max(N * d * 4, N * f * es));
  const size_t o_act_dxs = take("act_dxs", defer ? N * d * es : std::max(N * f * es, N * d * es));
  const size_t snf = align_up(N * f * es, 256), snd = align_up(N * d * es, 256);
  const size_t o_slot_act = take("slot_act", M * snf), o_slot_dh = take("slot_dh", M * snf);
  const size_t o_slot_dout = take("slot_dout", M * snd), o_slot_xs = take("slot_xs", M * snd);
  const size_t o_slot_cnt = take("slot_cnt", defer ? (size_t)moe::kMaxSlots * E * 4 : 0);
  const size_t o_slot_off = take("slot_off", defer ? (size_t)moe::kMaxSlots * E * 4 : 0);
  // G' [N, f]: not kept under the recomputation rule (the dH epilogue forms it from H)
  const bool recompute = (c.memory_rules & MOE_MEM_RECOMPUTE) != 0u;
  const size_t o_gp = take("gp", recompute ? 0 : N * f * es), o_dout = take("dout", N * d * es);
  const size_t o_wrt = take("wrt", (size_t)E * d * 4);
  const size_t o_rpart = take("rpart", rch * E * d * 4);
  const size_t o_loss = take("loss", (size_t)h.grid * 4);
  const size_t o_norm = take("norm", (size_t)(n10 + n11 + nrr) * 4);
  const size_t o_shadow = c.dtype == MOE_DTYPE_BF16 ? take("shadow", 2ull * E * d * f * 2) : 0;
  const size_t o_xs = c.dtype == MOE_DTYPE_BF16 ? take("xs", N * d * 2) : 0;
  // partial weight-gradient tiles of split contractions (skewed routing): at most
  // E/2 extra chunks over all experts (E in the applying launch of deferred
  // weight gradients), each a 128 x 128 fp32 tile per gradient tile; the
  // kernel never splits into more than the buffers hold
  const size_t wtiles = (size_t)cdiv(f, moe::gemm::BM) * cdiv(d, moe::gemm::BN);
  const size_t xchunks = c.max_microbatches > 1 ? (size_t)E + 1 : (size_t)E / 2 + 1;
  const size_t o_wpart2 = take("wpart2", xchunks * wtiles * moe::gemm::BM * moe::gemm::BN * 4);
  const size_t o_wpart1 = take("wpart1", xchunks * wtiles * moe::gemm::BM * moe::gemm::BN * 4);
  const int nrb = (int)((N + moe::gemm::BM - 1) / moe::gemm::BM) + E;   // row tiles of GEMM 1 (upper bound)
  const size_t o_ready = take("ready", (size_t)nrb * 4);
  if (base) {
    char* a = base;
    h.ctrl = reinterpret_cast<unsigned*>(a + o_ctrl);
    h.idx = reinterpret_cast<int*>(a + o_idx);
    h.gate = reinterpret_cast<float*>(a + o_gate);
    h.dzsel = reinterpret_cast<float*>(a + o_dz);
    h.hist = reinterpret_cast<int*>(a + o_hist);
    h.ready = reinterpret_cast<int*>(a + o_ready);
    h.nrb = nrb;
    h.perm = reinterpret_cast<int*>(a + o_perm);
    h.inv = reinterpret_cast<int*>(a + o_inv);
    h.act = a + o_act_dxs;
    h.gp = recompute ? a + o_act_dxs : a + o_gp;   // never read under the rule
    h.out = reinterpret_cast<float*>(a + o_out_dh);
    h.dout = a + o_dout;
    h.dh = a + o_out_dh;
    h.dxs = a + o_act_dxs;
    h.wrt = reinterpret_cast<float*>(a + o_wrt);
    h.rpart = reinterpret_cast<float*>(a + o_rpart);
    h.loss_part = reinterpret_cast<float*>(a + o_loss);
    h.norm_part = reinterpret_cast<float*>(a + o_norm);
    h.shadow = c.dtype == MOE_DTYPE_BF16 ? reinterpret_cast<uint16_t*>(a + o_shadow) : nullptr;
    h.xs = c.dtype == MOE_DTYPE_BF16 ? a + o_xs : nullptr;
    h.wpart2 = reinterpret_cast<float*>(a + o_wpart2);
    h.wpart1 = reinterpret_cast<float*>(a + o_wpart1);
    h.wpart_sets = (int)xchunks;
    if (defer) {
      h.slot_act = a + o_slot_act;
      h.slot_dh = a + o_slot_dh;
      h.slot_dout = a + o_slot_dout;
      h.slot_xs = a + o_slot_xs;
      h.stride_nf = (long)snf;
      h.stride_nd = (long)snd;
      h.slot_cnt = reinterpret_cast<int*>(a + o_slot_cnt);
      h.slot_off = reinterpret_cast<int*>(a + o_slot_off);
    }
  }
  return off;
}

// ---------------------------------------------------------------------------
// The arena of the allocation-free entry point: a static device array (each
// GPU the library runs on holds its own copy until the process ends).  The
// barrier words (for grids of up to 1003 workgroups) sit at its start, so no
// other call's buffers overlap them.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[MOE_STEP_STATIC_SCRATCH_BYTES];
constexpr size_t kStaticCtrlWords = 1024 * 32;   // grids of up to 1003 workgroups

// Before a static-arena launch: the barrier words, status and abort word of
// the previous call are cleared (a fill kernel, so the call stays one
// stream-ordered sequence of launches).
__global__ void static_clear(unsigned* ctrl, int words) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < words; i += gridDim.x * blockDim.x) ctrl[i] = 0u;
}

// After it: the device status bits of the launch into stats[3].
__global__ void static_report(const unsigned* status, float* stats) {
  if (threadIdx.x == 0) stats[3] = (float)*status;
}

struct StaticDevice {
  bool ready = false;
  char* ptr = nullptr;   // device address of this GPU's copy of `scratch`
  int cus = 0;
};
static std::mutex g_static_mu;
static StaticDevice g_static[64];

// Once per device, with that device current: the device address of its copy
// of the scratch array, its compute-unit count and architecture.
static int static_setup(int dev, char* err, StaticDevice** out) {
  std::lock_guard<std::mutex> lock(g_static_mu);
  StaticDevice& sd = g_static[dev];
  if (!sd.ready) {
    hipDeviceProp_t prop;
    hipError_t he = hipGetDeviceProperties(&prop, dev);
    if (he != hipSuccess) {
      set_err(err, "hipGetDeviceProperties: %s", hipGetErrorString(he));
      return MOE_ERR_HIP;
    }
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
      set_err(err, "device %d is %s; this library is built for gfx950 only", dev, prop.gcnArchName);
      return MOE_ERR_DEVICE;
    }
    void* ptr = nullptr;
    he = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (he != hipSuccess || !ptr) {
      set_err(err, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(he));
      return MOE_ERR_HIP;
    }
    sd.ptr = static_cast<char*>(ptr);
    sd.cus = prop.multiProcessorCount;
    sd.ready = true;
  }
  *out = &sd;
  return MOE_OK;
}

// Validates one launch's arguments (text into err) and enqueues the persistent
// kernel with h's arena.  Shared by the handle and static entry points.
static int run_impl(moe_step* h, char* err, const moe_step_io* io, int32_t n_tokens, int64_t tokens_in_update,
                    int64_t step_router, int64_t step_experts, uint32_t run_flags, void* hip_stream,
                    bool static_arena = false) {
  if (!io) {
    set_err(err, "io is NULL");
    return MOE_ERR_ARG;
  }
  const moe_step_config& c = h->cfg;
  if (n_tokens < 0 || n_tokens > c.max_tokens) {
    set_err(err, "n_tokens %d outside [0, max_tokens=%d]", n_tokens, c.max_tokens);
    return MOE_ERR_ARG;
  }
  if (tokens_in_update < 1 || tokens_in_update < n_tokens) {
    set_err(err, "tokens_in_update %lld must be >= max(1, n_tokens)", (long long)tokens_in_update);
    return MOE_ERR_ARG;
  }
  if (run_flags & ~(MOE_RUN_ZERO_GRAD | MOE_RUN_APPLY | MOE_RUN_REFRESH_SHADOW | MOE_RUN_TRACE | MOE_RUN_SKIP_MASK |
                    MOE_RUN_ZERO_GRAD_ROUTER | MOE_RUN_ZERO_GRAD_EXPERTS | MOE_RUN_APPLY_ROUTER |
                    MOE_RUN_APPLY_EXPERTS | MOE_RUN_READY_GEMM12 | MOE_RUN_COOPERATIVE | MOE_RUN_TEST_TIMEOUT |
                    MOE_RUN_BARRIER_PER_WORKGROUP)) {
    set_err(err, "unknown run flags 0x%x", run_flags);
    return MOE_ERR_ARG;
  }
  // the whole-update bits stand for both groups
  if (run_flags & MOE_RUN_ZERO_GRAD) run_flags |= MOE_RUN_ZERO_GRAD_ROUTER | MOE_RUN_ZERO_GRAD_EXPERTS;
  if (run_flags & MOE_RUN_APPLY) run_flags |= MOE_RUN_APPLY_ROUTER | MOE_RUN_APPLY_EXPERTS;
  run_flags &= ~(MOE_RUN_ZERO_GRAD | MOE_RUN_APPLY);
  const bool apply_r = (run_flags & MOE_RUN_APPLY_ROUTER) != 0u, apply_e = (run_flags & MOE_RUN_APPLY_EXPERTS) != 0u;
  if ((run_flags & MOE_RUN_SKIP_MASK) && h->last_full_tokens != n_tokens) {
    set_err(err, "skipping phases needs a previous full launch with the same n_tokens (%d, last %d)", n_tokens,
            h->last_full_tokens);
    return MOE_ERR_STATE;
  }
  if ((apply_r && step_router < 1) || (apply_e && step_experts < 1)) {
    set_err(err, "the AdamW step of an applied group must be >= 1 (router %lld, experts %lld)",
            (long long)step_router, (long long)step_experts);
    return MOE_ERR_ARG;
  }
  if (n_tokens > 0 && (!io->x || !io->target)) {
    set_err(err, "x and target are required");
    return MOE_ERR_ARG;
  }
  if (!io->params || !io->grads) {
    set_err(err, "params and grads are required");
    return MOE_ERR_ARG;
  }
  if ((apply_r || apply_e) && (!io->exp_avg || !io->exp_avg_sq)) {
    set_err(err, "exp_avg and exp_avg_sq are required with MOE_RUN_APPLY");
    return MOE_ERR_ARG;
  }
  if ((run_flags & MOE_RUN_TRACE) && !io->trace) {
    set_err(err, "MOE_RUN_TRACE needs io.trace");
    return MOE_ERR_ARG;
  }
  const uintptr_t mis = reinterpret_cast<uintptr_t>(io->x) | reinterpret_cast<uintptr_t>(io->target) |
                        reinterpret_cast<uintptr_t>(io->params) | reinterpret_cast<uintptr_t>(io->grads) |
                        reinterpret_cast<uintptr_t>(io->exp_avg) | reinterpret_cast<uintptr_t>(io->exp_avg_sq) |
                        reinterpret_cast<uintptr_t>(io->dx);
  if (mis & 15u) {
    set_err(err, "x, target, params, grads, exp_avg, exp_avg_sq and dx must be 16-byte aligned");
    return MOE_ERR_ARG;
  }

  moe::KParams p;
  std::memset(&p, 0, sizeof(p));
  p.T = n_tokens;
  p.d = c.d_model;
  p.f = c.d_ff;
  p.E = c.n_experts;
  p.k = c.top_k;
  p.inv_tupd = (float)(1.0 / (double)tokens_in_update);
  p.flags = run_flags;
  if (!h->shadow) p.flags &= ~MOE_RUN_REFRESH_SHADOW;
  p.lr = (float)c.lr;
  p.beta1 = (float)c.beta1;
  p.beta2 = (float)c.beta2;
  p.omb1 = (float)(1.0 - c.beta1);
  p.omb2 = (float)(1.0 - c.beta2);
  p.eps = (float)c.adam_eps;
  p.wd = (float)c.weight_decay;
  p.clip = (float)c.clip_norm;
  // bias corrections per group: [0] router, [1] experts
  const int64_t steps[2] = {step_router, step_experts};
  for (int q = 0; q < 2; ++q) {
    const double s = steps[q] >= 1 ? (double)steps[q] : 1.0;
    const double bc1 = 1.0 - std::pow(c.beta1, s), bc2 = 1.0 - std::pow(c.beta2, s);
    p.inv_bc1[q] = bc1 > 0.0 ? (float)(1.0 / bc1) : 1.f;
    p.inv_sqrt_bc2[q] = bc2 > 0.0 ? (float)(1.0 / std::sqrt(bc2)) : 1.f;
  }
  p.x = io->x;
  p.t = io->target;
  p.bias = io->router_bias;
  p.params = io->params;
  p.grads = io->grads;
  p.m = io->exp_avg;
  p.v = io->exp_avg_sq;
  p.dx = io->dx;
  p.stats = io->stats;
  p.dbg_logits = io->router_logits;
  p.dbg_idx = io->topk_idx;
  p.dbg_gate = io->topk_gate;
  p.dbg_counts = io->expert_counts;
  p.dbg_perm = io->route_perm;
  p.trace = io->trace;
  p.idx = h->idx;
  p.gate = h->gate;
  p.dzsel = h->dzsel;
  p.hist = h->hist;
  p.ready = h->ready;
  p.nrb = h->nrb;
  p.perm = h->perm;
  p.inv = h->inv;
  p.act = h->act;
  p.gp = h->gp;
  p.out = h->out;
  p.dout = h->dout;
  p.dh = h->dh;
  p.dxs = h->dxs;
  p.wrt = h->wrt;
  p.rpart = h->rpart;
  p.loss_part = h->loss_part;
  p.norm_part = h->norm_part;
  p.shadow = h->shadow;
  p.xs = h->xs;
  p.wpart2 = h->wpart2;
  p.wpart1 = h->wpart1;
  p.wpart_sets = h->wpart_sets;
  p.ctrl.gen = h->ctrl;
  p.ctrl.status = h->ctrl + 32;
  p.ctrl.abort = h->ctrl + 64;
  p.ctrl.arrive = h->ctrl + 128;
  p.ctrl.never = h->ctrl + 96;
  p.ctrl.xcd = h->ctrl + (size_t)(h->grid + 4) * 32;
  p.ctrl.per_wg = (run_flags & MOE_RUN_BARRIER_PER_WORKGROUP) ? 1 : 0;
  p.ctrl.limit = (run_flags & MOE_RUN_TEST_TIMEOUT) ? moe::kTestTimeoutTicks : moe::kBarrierTimeoutTicks;
  p.epoch = ++h->epoch;
  p.recompute = (c.memory_rules & MOE_MEM_RECOMPUTE) ? 1 : 0;
  p.nt_stores =
      (long)n_tokens * c.top_k >= (c.max_microbatches > 1 ? kNonTemporalRowsDeferred : kNonTemporalRows) ? 1 : 0;
  // deferred weight gradients: this launch's slot of the update
  int slot = -1;
  const bool zero_e = (run_flags & MOE_RUN_ZERO_GRAD_EXPERTS) != 0u;
  if (c.max_microbatches > 1) {
    if (static_arena || !h->slot_act) {
      set_err(err, "deferred weight gradients need a handle (max_microbatches > 1)");
      return MOE_ERR_ARG;
    }
    // (phase skipping stays available for profiling: route_order's offsets and
    // the slot tables are rebuilt by every launch from a histogram of the
    // same n_tokens, so every slot row stays within the arena)
    if (run_flags & MOE_RUN_TEST_TIMEOUT) {
      set_err(err, "the timeout test is not available with deferred weight gradients");
      return MOE_ERR_ARG;
    }
    slot = zero_e ? 0 : h->defer_slot + 1;
    if (slot >= c.max_microbatches) {
      set_err(err, "launch %d of an update whose experts are not applied yet; max_microbatches is %d", slot + 1,
              c.max_microbatches);
      return MOE_ERR_STATE;
    }
    p.defer = 1;
    p.slot = slot;
    p.defer_final = apply_e ? 1 : 0;
    p.defer_zero = (slot == 0 ? zero_e : h->defer_zero) ? 1 : 0;
    p.slot_act = h->slot_act;
    p.slot_dout = h->slot_dout;
    p.slot_xs = h->slot_xs;
    p.slot_dh = h->slot_dh;
    p.stride_nf = h->stride_nf;
    p.stride_nd = h->stride_nd;
    p.slot_cnt = h->slot_cnt;
    p.slot_off = h->slot_off;
    p.act = h->slot_act + (long)slot * h->stride_nf;
    p.dh = h->slot_dh + (long)slot * h->stride_nf;
    p.dout = h->slot_dout + (long)slot * h->stride_nd;
    p.xs = h->slot_xs + (long)slot * h->stride_nd;
  }

  hipError_t he = hipSetDevice(c.device);
  if (he != hipSuccess) {
    set_err(err, "hipSetDevice: %s", hipGetErrorString(he));
    return MOE_ERR_HIP;
  }
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  void* args[] = {&p};
  // The grid is exactly what the device holds at once, so an ordinary launch
  // makes it resident on an otherwise idle device; the cooperative launch
  // guarantees it but costs about 19 us more per update.
  const bool coop = (run_flags & MOE_RUN_COOPERATIVE) != 0u;
  if (static_arena) {
    hipLaunchKernelGGL(static_clear, dim3(16), dim3(256), 0, stream, h->ctrl, (int)ctrl_words(h->grid));
    if ((he = hipGetLastError()) != hipSuccess) {
      set_err(err, "clearing the barrier words: %s", hipGetErrorString(he));
      return MOE_ERR_HIP;
    }
  }
  he = coop ? hipLaunchCooperativeKernel(h->kern, dim3(h->grid), dim3(moe::kThreads), args, h->smem, stream)
            : hipLaunchKernel(h->kern, dim3(h->grid), dim3(moe::kThreads), args, h->smem, stream);
  if (he != hipSuccess) {
    set_err(err, "%s: %s", coop ? "hipLaunchCooperativeKernel" : "hipLaunchKernel", hipGetErrorString(he));
    return MOE_ERR_HIP;
  }
  if (static_arena) {
    hipLaunchKernelGGL(static_report, dim3(1), dim3(64), 0, stream, h->ctrl + 32, io->stats);
    if ((he = hipGetLastError()) != hipSuccess) {
      set_err(err, "reporting the device status: %s", hipGetErrorString(he));
      return MOE_ERR_HIP;
    }
  }
  h->last_stream = stream;
  h->launched = true;
  if (slot >= 0) {
    if (slot == 0) h->defer_zero = zero_e;
    h->defer_slot = apply_e ? -1 : slot;
  }
  if (run_flags & MOE_RUN_TEST_TIMEOUT) h->last_full_tokens = -1;
  else if (!(run_flags & MOE_RUN_SKIP_MASK)) h->last_full_tokens = n_tokens;
  return MOE_OK;
}

extern "C" {

size_t moe_step_param_count(const moe_step_config* c) {
  if (!c) return 0;
  return (size_t)c->d_model * c->n_experts + 2ull * c->n_experts * c->d_model * c->d_ff;
}

int moe_step_check_config(const moe_step_config* cfg) {
  char err[512];
  return check_config(cfg, err);
}

const char* moe_step_last_error(moe_step_t h) { return h ? h->err : g_create_error; }

int moe_step_grid_size(moe_step_t h) { return h ? h->grid : 0; }

size_t moe_step_arena_bytes(moe_step_t h) { return h ? h->arena_bytes : 0; }

size_t moe_step_trace_words(moe_step_t h) { return h ? (size_t)h->grid * moe::kPhases * 3 : 0; }

int moe_step_create(const moe_step_config* cfg, moe_step_t* out) {
  if (!out) {
    set_err(g_create_error, "out is NULL");
    return MOE_ERR_ARG;
  }
  *out = nullptr;
  int rc = check_config(cfg, g_create_error);
  if (rc != MOE_OK) return rc;

  int ndev = 0;
  hipError_t he = hipGetDeviceCount(&ndev);
  if (he != hipSuccess || ndev <= 0) {
    set_err(g_create_error, "no HIP device (%s)", hipGetErrorString(he));
    return MOE_ERR_HIP;
  }
  if (cfg->device < 0 || cfg->device >= ndev) {
    set_err(g_create_error, "device %d out of range (%d devices)", cfg->device, ndev);
    return MOE_ERR_ARG;
  }
  if ((he = hipSetDevice(cfg->device)) != hipSuccess) {
    set_err(g_create_error, "hipSetDevice: %s", hipGetErrorString(he));
    return MOE_ERR_HIP;
  }
  hipDeviceProp_t prop;
  if ((he = hipGetDeviceProperties(&prop, cfg->device)) != hipSuccess) {
    set_err(g_create_error, "hipGetDeviceProperties: %s", hipGetErrorString(he));
    return MOE_ERR_HIP;
  }
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    set_err(g_create_error, "device %d is %s; this library is built for gfx950 only", cfg->device,
            prop.gcnArchName);
    return MOE_ERR_DEVICE;
  }
  if (!prop.cooperativeLaunch) {
    set_err(g_create_error, "device does not support cooperative launches");
    return MOE_ERR_DEVICE;
  }

  moe_step* h = new (std::nothrow) moe_step();
  if (!h) {
    set_err(g_create_error, "host allocation failed");
    return MOE_ERR_NOMEM;
  }
  h->cfg = *cfg;
  if ((rc = select_kernel(*cfg, prop.multiProcessorCount, *h, g_create_error)) != MOE_OK) {
    delete h;
    return rc;
  }
  h->arena_bytes = plan_arena(*h, nullptr, ctrl_words(h->grid));

  he = hipMalloc(reinterpret_cast<void**>(&h->arena), h->arena_bytes);
  if (he != hipSuccess) {
    set_err(g_create_error, "hipMalloc(%zu bytes): %s", h->arena_bytes, hipGetErrorString(he));
    delete h;
    return MOE_ERR_NOMEM;
  }
  plan_arena(*h, h->arena, ctrl_words(h->grid));

  // the arena starts zeroed (every stored index is then in range) and so do
  // the barrier words and status (synchronous; not part of any run)
  he = hipMemset(h->arena, 0, h->arena_bytes);
  if (he == hipSuccess) he = hipDeviceSynchronize();
  if (he != hipSuccess) {
    set_err(g_create_error, "clearing barrier words: %s", hipGetErrorString(he));
    (void)hipFree(h->arena);
    delete h;
    return MOE_ERR_HIP;
  }
  *out = h;
  return MOE_OK;
}

int moe_step_run(moe_step_t h, const moe_step_io* io, int32_t n_tokens, int64_t tokens_in_update, int64_t step,
                 uint32_t run_flags, void* hip_stream) {
  return moe_step_run_groups(h, io, n_tokens, tokens_in_update, step, step, run_flags, hip_stream);
}

int moe_step_run_groups(moe_step_t h, const moe_step_io* io, int32_t n_tokens, int64_t tokens_in_update,
                        int64_t step_router, int64_t step_experts, uint32_t run_flags, void* hip_stream) {
  if (!h) return MOE_ERR_ARG;
  return run_impl(h, h->err, io, n_tokens, tokens_in_update, step_router, step_experts, run_flags, hip_stream);
}

int moe_step_run_static(const moe_step_config* cfg, const moe_step_io* io, int32_t n_tokens,
                        int64_t tokens_in_update, int64_t step, uint32_t run_flags, void* hip_stream) {
  char* err = g_create_error;
  int rc = check_config(cfg, err);
  if (rc != MOE_OK) return rc;
  if (!io || !io->stats) {
    set_err(err, "io and io->stats are required (stats[3] receives the device status)");
    return MOE_ERR_ARG;
  }
  if (cfg->memory_rules & MOE_MEM_GUARDS) {
    set_err(err, "MOE_MEM_GUARDS needs a handle (moe_step_check_guards reads its zones)");
    return MOE_ERR_ARG;
  }
  if (run_flags & MOE_RUN_SKIP_MASK) {
    set_err(err, "phase skipping needs a handle (it reuses the previous launch's arena)");
    return MOE_ERR_ARG;
  }
  int ndev = 0;
  hipError_t he = hipGetDeviceCount(&ndev);
  if (he != hipSuccess || ndev <= 0) {
    set_err(err, "no HIP device (%s)", hipGetErrorString(he));
    return MOE_ERR_HIP;
  }
  if (cfg->device < 0 || cfg->device >= ndev || cfg->device >= 64) {
    set_err(err, "device %d out of range (%d devices)", cfg->device, ndev);
    return MOE_ERR_ARG;
  }
  if ((he = hipSetDevice(cfg->device)) != hipSuccess) {
    set_err(err, "hipSetDevice: %s", hipGetErrorString(he));
    return MOE_ERR_HIP;
  }
  StaticDevice* sd = nullptr;
  if ((rc = static_setup(cfg->device, err, &sd)) != MOE_OK) return rc;
  moe_step h;   // on the stack: the handle state of this one call
  h.cfg = *cfg;
  if ((rc = select_kernel(*cfg, sd->cus, h, err)) != MOE_OK) return rc;
  if (ctrl_words(h.grid) > kStaticCtrlWords) {
    set_err(err, "grid of %d workgroups exceeds the static barrier words", h.grid);
    return MOE_ERR_SHAPE;
  }
  const size_t need = plan_arena(h, nullptr, kStaticCtrlWords);
  if (need > (size_t)MOE_STEP_STATIC_SCRATCH_BYTES) {
    set_err(err, "this configuration needs %zu bytes of arena; the static scratch holds %zu", need,
            (size_t)MOE_STEP_STATIC_SCRATCH_BYTES);
    return MOE_ERR_SHAPE;
  }
  plan_arena(h, sd->ptr, kStaticCtrlWords);
  h.arena_bytes = need;
  // the array is shared by every call on this GPU, so the bf16 weight copy is
  // always rebuilt from params
  return run_impl(&h, err, io, n_tokens, tokens_in_update, step, step, run_flags | MOE_RUN_REFRESH_SHADOW,
                  hip_stream, true);
}

int moe_step_status(moe_step_t h) {
  if (!h) return MOE_ERR_ARG;
  hipError_t he = hipSetDevice(h->cfg.device);
  if (he == hipSuccess && h->launched) he = hipStreamSynchronize(h->last_stream);
  if (he != hipSuccess) {
    set_err(h->err, "waiting for the stream: %s", hipGetErrorString(he));
    return MOE_ERR_HIP;
  }
  unsigned st = 0;
  he = hipMemcpy(&st, h->ctrl + 32, sizeof(unsigned), hipMemcpyDeviceToHost);
  if (he != hipSuccess) {
    set_err(h->err, "reading the status word: %s", hipGetErrorString(he));
    return MOE_ERR_HIP;
  }
  if (st != 0u) {
    set_err(h->err, "device error 0x%x:%s%s%s", st, (st & MOE_DEVICE_BARRIER_TIMEOUT) ? " grid-barrier timeout" : "",
            (st & MOE_DEVICE_NONFINITE_LOGIT) ? " non-finite router logit" : "",
            (st & MOE_DEVICE_BAD_ROUTE) ? " expert index out of range" : "");
    he = hipMemset(h->ctrl, 0, ctrl_words(h->grid) * sizeof(unsigned));
    if (he == hipSuccess) he = hipDeviceSynchronize();
    h->epoch = 0;
    return MOE_ERR_DEVICE;
  }
  return MOE_OK;
}

int moe_step_check_guards(moe_step_t h, int32_t* damaged) {
  if (damaged) *damaged = 0;
  if (!h) return MOE_ERR_ARG;
  if (!(h->cfg.memory_rules & MOE_MEM_GUARDS)) {
    set_err(h->err, "the handle was created without MOE_MEM_GUARDS");
    return MOE_ERR_STATE;
  }
  hipError_t he = hipSetDevice(h->cfg.device);
  if (he == hipSuccess && h->launched) he = hipStreamSynchronize(h->last_stream);
  if (he != hipSuccess) {
    set_err(h->err, "waiting for the stream: %s", hipGetErrorString(he));
    return MOE_ERR_HIP;
  }
  size_t most = 0;
  for (int i = 0; i < h->n_guards; ++i) most = std::max(most, h->guards[i].len);
  unsigned char* buf = new (std::nothrow) unsigned char[most];
  if (!buf) {
    set_err(h->err, "host allocation failed");
    return MOE_ERR_NOMEM;
  }
  int bad = 0;
  const char* first = nullptr;
  size_t first_at = 0;
  for (int i = 0; i < h->n_guards; ++i) {
    const moe_step::Guard& g = h->guards[i];
    he = hipMemcpy(buf, h->arena + g.off, g.len, hipMemcpyDeviceToHost);
    if (he != hipSuccess) {
      delete[] buf;
      set_err(h->err, "reading a guard zone: %s", hipGetErrorString(he));
      return MOE_ERR_HIP;
    }
    for (size_t b = 0; b < g.len; ++b)
      if (buf[b] != 0) {
        if (!first) {
          first = g.after;
          first_at = b;
        }
        ++bad;
        break;
      }
  }
  delete[] buf;
  if (damaged) *damaged = bad;
  if (bad) {
    set_err(h->err, "%d guard zone(s) written; the first follows arena buffer %s (byte %zu past its end)", bad,
            first, first_at);
    return MOE_ERR_STATE;
  }
  return MOE_OK;
}

void moe_step_destroy(moe_step_t h) {
  if (!h) return;
  if (hipSetDevice(h->cfg.device) == hipSuccess) {
    if (h->launched) (void)hipStreamSynchronize(h->last_stream);
    if (h->arena) (void)hipFree(h->arena);
  }
  delete h;
}

}  // extern "C"
