// moe_step_bench: drives the C ABI of libmoe_step from C++ alone (no Python),
// for profiling runs under rocprofv3 and as an example of the ABI.
//
// Inputs: with --inputs FILE, exactly the seeded inputs of the tests and the
// Python bench (written by `python -m synth.dump`), including the number of
// microbatches of the update and the router bias; otherwise synthetic inputs
// shaped like the layer workloads (x, t ~ N(0,1), weights ~ N(0, 0.02^2) from a
// splitmix64 generator and a Box-Muller transform).  One timed unit is one
// update: its microbatches in order, the first with MOE_RUN_ZERO_GRAD, the
// last with MOE_RUN_APPLY.  Prints one line per skip mask with ms/update.
//
//   moe_step_bench [--config NAME | --inputs FILE] [--steps K] [--warmup W] [--skip MASK[,MASK...]]
//                  [--wg-per-cu N] [--ready] [--coop] [--recompute] [--per-wg-barrier] [--fresh] [--defer]
//                  [--copy-mib N]
//     NAME: tiny_f32 | bf16_2x1024 | bf16_32x1024 | top8_4x1024 (--tokens N changes its token count)
//     --skip MASK: after the warm-up, time K updates whose launches skip the
//                  phases in MASK (bit i = phase i, 0..7; bit 8 = the dispatch
//                  gather inside phase 1; bit 9 = the k-way row sum of dx inside
//                  phase 7), for per-phase timing and counter collection; a
//                  comma-separated list times K updates per mask, in order
//     --fresh: every update (warm-up and timed) starts from the initial
//              parameters and zero moments at step 1, restored on the stream
//              before its first launch and outside its timing (events around
//              each update's launches), so every update routes like the first;
//              without it the parameters keep training from update to update
//     --defer: deferred expert weight gradients (max_microbatches = the
//              update's microbatch count, when more than one)
//     --copy-mib N: instead, time a plain device copy of N MiB (read N, write N),
//                  the reference for scaling memory counters
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/moe_step.h"

#define CHECK_HIP(x)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (x);                                                               \
    if (e_ != hipSuccess) {                                                            \
      std::fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
      std::exit(2);                                                                    \
    }                                                                                  \
  } while (0)

namespace {

struct Shape {
  const char* name;
  int T, d, f, E, k;
  int dtype;
  int M = 1;   // microbatches per update
};

const Shape kShapes[] = {
    {"tiny_f32", 256, 64, 128, 4, 2, MOE_DTYPE_F32},
    {"bf16_2x1024", 2048, 768, 1536, 16, 2, MOE_DTYPE_BF16},
    {"bf16_32x1024", 32768, 768, 1536, 16, 2, MOE_DTYPE_BF16},
    {"top8_4x1024", 4096, 1024, 512, 64, 8, MOE_DTYPE_BF16},
};

struct Rng {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
  }
  double uniform() { return ((next() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }
  double normal() {
    const double u1 = uniform(), u2 = uniform();
    return std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586 * u2);
  }
};

uint16_t to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ void copy_kernel(const float4* __restrict__ a, float4* __restrict__ b, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += stride) b[i] = a[i];
}

int run_copy(int mib, int steps) {
  const size_t n4 = ((size_t)mib << 20) / 16;
  float4 *a, *b;
  CHECK_HIP(hipMalloc(&a, n4 * 16));
  CHECK_HIP(hipMalloc(&b, n4 * 16));
  CHECK_HIP(hipMemset(a, 0, n4 * 16));
  hipEvent_t e0, e1;
  CHECK_HIP(hipEventCreate(&e0));
  CHECK_HIP(hipEventCreate(&e1));
  copy_kernel<<<4096, 256>>>(a, b, n4);
  CHECK_HIP(hipEventRecord(e0));
  for (int i = 0; i < steps; ++i) copy_kernel<<<4096, 256>>>(a, b, n4);
  CHECK_HIP(hipEventRecord(e1));
  CHECK_HIP(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK_HIP(hipEventElapsedTime(&ms, e0, e1));
  std::printf("copy %d MiB: %.4f ms per copy, %.1f GB/s (read+write)\n", mib, ms / steps,
              2.0 * n4 * 16 * steps / (ms * 1e-3) / 1e9);
  CHECK_HIP(hipFree(a));
  CHECK_HIP(hipFree(b));
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  std::string cfg_name = "bf16_2x1024", inputs;
  int tokens = 0;   // --tokens: tokens per launch for a built-in shape (0 = the shape's own)
  int steps = 20, warmup = 3, copy_mib = 0, wg_per_cu = 0;
  bool ready = false, coop = false, recompute = false, per_wg = false, fresh = false, defer = false;
  std::vector<unsigned> skips{0u};
  for (int i = 1; i < argc; ++i) {
    std::string a = argv[i];
    auto next = [&]() -> const char* {
      if (i + 1 >= argc) {
        std::fprintf(stderr, "missing value for %s\n", a.c_str());
        std::exit(1);
      }
      return argv[++i];
    };
    if (a == "--config") cfg_name = next();
    else if (a == "--inputs") inputs = next();
    else if (a == "--tokens") tokens = std::atoi(next());
    else if (a == "--steps") steps = std::atoi(next());
    else if (a == "--warmup") warmup = std::atoi(next());
    else if (a == "--skip") {
      skips.clear();
      std::string s = next();
      size_t pos = 0;
      while (pos <= s.size()) {
        const size_t q = s.find(',', pos);
        skips.push_back((unsigned)std::strtoul(s.substr(pos, q == std::string::npos ? std::string::npos : q - pos).c_str(), nullptr, 0));
        if (q == std::string::npos) break;
        pos = q + 1;
      }
    }
    else if (a == "--copy-mib") copy_mib = std::atoi(next());
    else if (a == "--wg-per-cu") wg_per_cu = std::atoi(next());
    else if (a == "--ready") ready = true;
    else if (a == "--coop") coop = true;
    else if (a == "--recompute") recompute = true;
    else if (a == "--per-wg-barrier") per_wg = true;
    else if (a == "--fresh") fresh = true;
    else if (a == "--defer") defer = true;
    else {
      std::fprintf(stderr, "unknown argument %s\n", a.c_str());
      return 1;
    }
  }
  if (copy_mib > 0) return run_copy(copy_mib, steps);

  Shape file_shape{"inputs", 0, 0, 0, 0, 0, 0};
  std::vector<char> hx, ht;
  std::vector<float> hp, hbias;
  const Shape* sh = nullptr;
  if (!inputs.empty()) {
    // the seeded inputs of the tests (synth.dump)
    FILE* fh = std::fopen(inputs.c_str(), "rb");
    if (!fh) {
      std::fprintf(stderr, "cannot open %s\n", inputs.c_str());
      return 1;
    }
    char magic[8];
    int32_t hd[8];
    if (std::fread(magic, 1, 8, fh) != 8 || std::memcmp(magic, "MOEIN001", 8) != 0 ||
        std::fread(hd, 4, 8, fh) != 8) {
      std::fprintf(stderr, "%s is not an input file of synth.dump\n", inputs.c_str());
      return 1;
    }
    file_shape = Shape{"inputs", hd[0], hd[2], hd[3], hd[4], hd[5], hd[6] ? MOE_DTYPE_BF16 : MOE_DTYPE_F32, hd[1]};
    const size_t es = hd[6] ? 2 : 4;
    const size_t nx = (size_t)hd[0] * hd[1] * hd[2];
    const size_t P = (size_t)hd[2] * hd[4] + 2ull * hd[4] * hd[2] * hd[3];
    hx.resize(nx * es);
    ht.resize(nx * es);
    hp.resize(P);
    bool ok = std::fread(hx.data(), 1, hx.size(), fh) == hx.size() && std::fread(ht.data(), 1, ht.size(), fh) == ht.size() &&
              std::fread(hp.data(), 4, P, fh) == P;
    if (ok && hd[7]) {
      hbias.resize(hd[4]);
      ok = std::fread(hbias.data(), 4, hbias.size(), fh) == hbias.size();
    }
    std::fclose(fh);
    if (!ok) {
      std::fprintf(stderr, "%s is truncated\n", inputs.c_str());
      return 1;
    }
    sh = &file_shape;
  } else {
    for (const Shape& s : kShapes)
      if (cfg_name == s.name) sh = &s;
    if (!sh) {
      std::fprintf(stderr, "unknown config %s\n", cfg_name.c_str());
      return 1;
    }
    if (tokens > 0) {
      file_shape = *sh;
      file_shape.T = tokens;
      sh = &file_shape;
    }
  }
  const int M = sh->M;
  moe_step_config cfg;
  std::memset(&cfg, 0, sizeof(cfg));
  cfg.struct_size = sizeof(cfg);
  cfg.abi_version = MOE_STEP_ABI_VERSION;
  cfg.d_model = sh->d;
  cfg.d_ff = sh->f;
  cfg.n_experts = sh->E;
  cfg.top_k = sh->k;
  cfg.max_tokens = sh->T;
  cfg.dtype = sh->dtype;
  cfg.lr = 1e-3;
  cfg.beta1 = 0.9;
  cfg.beta2 = 0.999;
  cfg.adam_eps = 1e-8;
  cfg.weight_decay = 0.01;
  cfg.clip_norm = 1.0;
  cfg.wg_per_cu = wg_per_cu;
  cfg.memory_rules = recompute ? MOE_MEM_RECOMPUTE : 0u;
  cfg.max_microbatches = defer && M > 1 ? M : 0;
  moe_step_t h = nullptr;
  if (moe_step_create(&cfg, &h) != MOE_OK) {
    std::fprintf(stderr, "moe_step_create: %s\n", moe_step_last_error(nullptr));
    return 2;
  }
  const size_t P = moe_step_param_count(&cfg);
  const size_t nt = (size_t)sh->T * sh->d;   // elements of one microbatch's x
  const size_t es = sh->dtype == MOE_DTYPE_BF16 ? 2 : 4;
  if (inputs.empty()) {
    Rng rng{0x5eedull};
    hp.resize(P);
    for (size_t i = 0; i < P; ++i) hp[i] = (float)(0.02 * rng.normal());
    hx.resize(nt * es);
    ht.resize(nt * es);
    for (std::vector<char>* v : {&hx, &ht})
      for (size_t i = 0; i < nt; ++i) {
        const float a = (float)rng.normal();
        if (es == 2) {
          const uint16_t b = to_bf16(a);
          std::memcpy(&(*v)[i * 2], &b, 2);
        } else {
          std::memcpy(&(*v)[i * 4], &a, 4);
        }
      }
  }
  char *dx_in, *dt;
  float *params, *grads, *m, *v, *dxg, *stats, *bias = nullptr;
  CHECK_HIP(hipMalloc(&dx_in, hx.size()));
  CHECK_HIP(hipMalloc(&dt, ht.size()));
  CHECK_HIP(hipMalloc(&params, P * 4));
  CHECK_HIP(hipMalloc(&grads, P * 4));
  CHECK_HIP(hipMalloc(&m, P * 4));
  CHECK_HIP(hipMalloc(&v, P * 4));
  CHECK_HIP(hipMalloc(&dxg, nt * 4));
  CHECK_HIP(hipMalloc(&stats, 16));
  CHECK_HIP(hipMemcpy(dx_in, hx.data(), hx.size(), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dt, ht.data(), ht.size(), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(params, hp.data(), P * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemset(m, 0, P * 4));
  CHECK_HIP(hipMemset(v, 0, P * 4));
  if (!hbias.empty()) {
    CHECK_HIP(hipMalloc(&bias, hbias.size() * 4));
    CHECK_HIP(hipMemcpy(bias, hbias.data(), hbias.size() * 4, hipMemcpyHostToDevice));
  }

  moe_step_io io;
  std::memset(&io, 0, sizeof(io));
  io.params = params;
  io.grads = grads;
  io.exp_avg = m;
  io.exp_avg_sq = v;
  io.dx = dxg;
  io.stats = stats;
  io.router_bias = bias;
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  const uint32_t base = (ready ? MOE_RUN_READY_GEMM12 : 0u) | (coop ? MOE_RUN_COOPERATIVE : 0u) |
                        (per_wg ? MOE_RUN_BARRIER_PER_WORKGROUP : 0u);
  int64_t step = 1;
  bool first = true;
  // --fresh: the initial parameters, restored before every update
  float* params0 = nullptr;
  if (fresh) {
    CHECK_HIP(hipMalloc(&params0, P * 4));
    CHECK_HIP(hipMemcpy(params0, params, P * 4, hipMemcpyDeviceToDevice));
  }
  // one update: the microbatches in order (x and t of microbatch mb at offset mb * T);
  // with --fresh, e0/e1 (when given) bracket its launches and not the restore
  auto update = [&](uint32_t extra, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr) -> int {
    if (fresh) {
      CHECK_HIP(hipMemcpyAsync(params, params0, P * 4, hipMemcpyDeviceToDevice, stream));
      CHECK_HIP(hipMemsetAsync(m, 0, P * 4, stream));
      CHECK_HIP(hipMemsetAsync(v, 0, P * 4, stream));
      step = 1;
    }
    if (ev0) CHECK_HIP(hipEventRecord(ev0, stream));
    for (int mb = 0; mb < M; ++mb) {
      io.x = dx_in + (size_t)mb * nt * es;
      io.target = dt + (size_t)mb * nt * es;
      uint32_t fl = base | extra | (mb == 0 ? MOE_RUN_ZERO_GRAD : 0u) | (mb == M - 1 ? MOE_RUN_APPLY : 0u);
      if (first) fl |= MOE_RUN_REFRESH_SHADOW;
      first = false;
      if (moe_step_run(h, &io, sh->T, (int64_t)sh->T * M, step, fl, stream) != MOE_OK) {
        std::fprintf(stderr, "moe_step_run: %s\n", moe_step_last_error(h));
        return 2;
      }
    }
    if (ev1) CHECK_HIP(hipEventRecord(ev1, stream));
    ++step;
    return 0;
  };
  for (int i = 0; i < warmup; ++i)
    if (update(0u)) return 2;
  if (moe_step_status(h) != MOE_OK) {
    std::fprintf(stderr, "moe_step_status: %s\n", moe_step_last_error(h));
    return 2;
  }
  hipEvent_t e0, e1;
  CHECK_HIP(hipEventCreate(&e0));
  CHECK_HIP(hipEventCreate(&e1));
  std::vector<hipEvent_t> fe(fresh ? 2 * (size_t)std::max(steps, 1) : 0);
  for (hipEvent_t& e : fe) CHECK_HIP(hipEventCreate(&e));
  if (steps < 1) {
    std::fprintf(stderr, "--steps must be at least 1\n");
    return 1;
  }
  for (const unsigned skip : skips) {
    const uint32_t sk = ((skip & 0xffu) << 8) | ((skip & 0x100u) ? MOE_RUN_SKIP_GATHER : 0u) |
                        ((skip & 0x200u) ? MOE_RUN_SKIP_ROWSUM : 0u);
    float ms = 0.f;
    if (fresh) {
      // events around each update's launches; the restores stay outside them
      for (int i = 0; i < steps; ++i) {
        if (update(sk, fe[2 * i], fe[2 * i + 1])) return 2;
      }
      CHECK_HIP(hipEventSynchronize(fe[2 * steps - 1]));
      for (int i = 0; i < steps; ++i) {
        float u = 0.f;
        CHECK_HIP(hipEventElapsedTime(&u, fe[2 * i], fe[2 * i + 1]));
        ms += u;
      }
    } else {
      CHECK_HIP(hipEventRecord(e0, stream));
      for (int i = 0; i < steps; ++i)
        if (update(sk)) return 2;
      CHECK_HIP(hipEventRecord(e1, stream));
      CHECK_HIP(hipEventSynchronize(e1));
      CHECK_HIP(hipEventElapsedTime(&ms, e0, e1));
    }
    if (moe_step_status(h) != MOE_OK) {
      std::fprintf(stderr, "moe_step_status: %s\n", moe_step_last_error(h));
      return 2;
    }
    std::printf("%s skip=0x%03x grid=%d: %d %supdates of %d launch(es), %.4f ms/update, %.0f tokens/s\n",
                inputs.empty() ? sh->name : inputs.c_str(), skip, moe_step_grid_size(h), steps, fresh ? "fresh " : "",
                M, ms / steps, (double)sh->T * M * steps / (ms * 1e-3));
    std::fflush(stdout);
  }
  for (hipEvent_t e : fe) CHECK_HIP(hipEventDestroy(e));
  if (params0) CHECK_HIP(hipFree(params0));
  moe_step_destroy(h);
  for (void* p : {(void*)dx_in, (void*)dt, (void*)params, (void*)grads, (void*)m, (void*)v, (void*)dxg, (void*)stats})
    CHECK_HIP(hipFree(p));
  if (bias) CHECK_HIP(hipFree(bias));
  CHECK_HIP(hipStreamDestroy(stream));
  return 0;
}
