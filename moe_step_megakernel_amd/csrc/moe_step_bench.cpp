// moe_step_bench: drives the C ABI of libmoe_step from C++ alone (no Python),
// for profiling runs under rocprofv3 and as an example of the ABI.
//
// Inputs are synthetic and shaped like the layer workloads: x, t ~ N(0,1) and
// weights ~ N(0, 0.02^2), drawn with a splitmix64 generator and a Box-Muller
// transform (a different stream from the Python generator; timings do not
// depend on the exact values).  Prints one line per run with ms/update.
//
//   moe_step_bench [--config NAME] [--steps K] [--warmup W] [--skip MASK[,MASK...]] [--wg-per-cu N] [--ready]
//                  [--coop] [--copy-mib N]
//     NAME: tiny_f32 | bf16_2x1024 | bf16_32x1024 | top8_4x1024
//     --skip MASK: after the warm-up, time K launches that skip the phases in MASK
//                  (bit i = phase i), for per-phase timing and counter collection;
//                  a comma-separated list times K launches per mask, in order
//     --copy-mib N: instead, time a plain device copy of N MiB (read N, write N),
//                  the reference for scaling memory counters
#include <hip/hip_runtime.h>

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
  std::string cfg_name = "bf16_2x1024";
  int steps = 20, warmup = 3, copy_mib = 0, wg_per_cu = 0;
  bool ready = false, coop = false, recompute = false, per_wg = false;
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
    else {
      std::fprintf(stderr, "unknown argument %s\n", a.c_str());
      return 1;
    }
  }
  if (copy_mib > 0) return run_copy(copy_mib, steps);

  const Shape* sh = nullptr;
  for (const Shape& s : kShapes)
    if (cfg_name == s.name) sh = &s;
  if (!sh) {
    std::fprintf(stderr, "unknown config %s\n", cfg_name.c_str());
    return 1;
  }
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
  moe_step_t h = nullptr;
  if (moe_step_create(&cfg, &h) != MOE_OK) {
    std::fprintf(stderr, "moe_step_create: %s\n", moe_step_last_error(nullptr));
    return 2;
  }
  const size_t P = moe_step_param_count(&cfg);
  const size_t nx = (size_t)sh->T * sh->d;
  const size_t es = sh->dtype == MOE_DTYPE_BF16 ? 2 : 4;
  Rng rng{0x5eedull};
  std::vector<float> hp(P);
  for (size_t i = 0; i < P; ++i) hp[i] = (float)(0.02 * rng.normal());
  std::vector<char> hx(nx * es), ht(nx * es);
  for (size_t i = 0; i < nx; ++i) {
    const float a = (float)rng.normal();
    if (es == 2) {
      const uint16_t b = to_bf16(a);
      std::memcpy(&hx[i * 2], &b, 2);
    } else {
      std::memcpy(&hx[i * 4], &a, 4);
    }
  }
  for (size_t i = 0; i < nx; ++i) {
    const float a = (float)rng.normal();
    if (es == 2) {
      const uint16_t b = to_bf16(a);
      std::memcpy(&ht[i * 2], &b, 2);
    } else {
      std::memcpy(&ht[i * 4], &a, 4);
    }
  }
  void *dx_in, *dt;
  float *params, *grads, *m, *v, *dxg, *stats;
  CHECK_HIP(hipMalloc(&dx_in, nx * es));
  CHECK_HIP(hipMalloc(&dt, nx * es));
  CHECK_HIP(hipMalloc(&params, P * 4));
  CHECK_HIP(hipMalloc(&grads, P * 4));
  CHECK_HIP(hipMalloc(&m, P * 4));
  CHECK_HIP(hipMalloc(&v, P * 4));
  CHECK_HIP(hipMalloc(&dxg, nx * 4));
  CHECK_HIP(hipMalloc(&stats, 16));
  CHECK_HIP(hipMemcpy(dx_in, hx.data(), nx * es, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dt, ht.data(), nx * es, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(params, hp.data(), P * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemset(m, 0, P * 4));
  CHECK_HIP(hipMemset(v, 0, P * 4));

  moe_step_io io;
  std::memset(&io, 0, sizeof(io));
  io.x = dx_in;
  io.target = dt;
  io.params = params;
  io.grads = grads;
  io.exp_avg = m;
  io.exp_avg_sq = v;
  io.dx = dxg;
  io.stats = stats;
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  const uint32_t base =
      MOE_RUN_ZERO_GRAD | MOE_RUN_APPLY | (ready ? MOE_RUN_READY_GEMM12 : 0u) | (coop ? MOE_RUN_COOPERATIVE : 0u) |
      (per_wg ? MOE_RUN_BARRIER_PER_WORKGROUP : 0u);
  int64_t step = 1;
  for (int i = 0; i < warmup; ++i, ++step) {
    if (moe_step_run(h, &io, sh->T, sh->T, step, base | (i == 0 ? MOE_RUN_REFRESH_SHADOW : 0u), stream) != MOE_OK) {
      std::fprintf(stderr, "moe_step_run: %s\n", moe_step_last_error(h));
      return 2;
    }
  }
  if (moe_step_status(h) != MOE_OK) {
    std::fprintf(stderr, "moe_step_status: %s\n", moe_step_last_error(h));
    return 2;
  }
  hipEvent_t e0, e1;
  CHECK_HIP(hipEventCreate(&e0));
  CHECK_HIP(hipEventCreate(&e1));
  for (const unsigned skip : skips) {
    CHECK_HIP(hipEventRecord(e0, stream));
    for (int i = 0; i < steps; ++i, ++step) {
      if (moe_step_run(h, &io, sh->T, sh->T, step, base | (skip << 8), stream) != MOE_OK) {
        std::fprintf(stderr, "moe_step_run: %s\n", moe_step_last_error(h));
        return 2;
      }
    }
    CHECK_HIP(hipEventRecord(e1, stream));
    CHECK_HIP(hipEventSynchronize(e1));
    if (moe_step_status(h) != MOE_OK) {
      std::fprintf(stderr, "moe_step_status: %s\n", moe_step_last_error(h));
      return 2;
    }
    float ms = 0.f;
    CHECK_HIP(hipEventElapsedTime(&ms, e0, e1));
    std::printf("%s skip=0x%02x grid=%d: %d updates, %.4f ms/update, %.0f tokens/s\n", sh->name, skip,
                moe_step_grid_size(h), steps, ms / steps, sh->T * steps / (ms * 1e-3));
    std::fflush(stdout);
  }
  moe_step_destroy(h);
  for (void* p : {dx_in, dt, (void*)params, (void*)grads, (void*)m, (void*)v, (void*)dxg, (void*)stats})
    CHECK_HIP(hipFree(p));
  CHECK_HIP(hipStreamDestroy(stream));
  return 0;
}
