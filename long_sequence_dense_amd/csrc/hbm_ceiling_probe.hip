// HBM streaming rates this GPU sustains for plain passes over one tensor of
// the Q/K prep's inputs ([40, 109000, 128] BF16, 1.116 GB): the ceilings
// against which the prep's memory-bound kernels are read.
//
// Passes (each with 16-byte accesses; a wave's load or store instruction
// covers 1 KB of consecutive bytes):
//   read        read-only (an XOR of every word; one word written per
//               workgroup only if the XOR hits a fixed value, which it never
//               does for the fill used here), ordinary and non-temporal loads;
//   copy        read + write of the same size, ordinary and non-temporal loads;
//   write       write-only of the code and scale bytes of one prepared tensor
//               (0.314 GB).
// Launch shapes: one workgroup of 256 threads per 256 x U vectors (U = 1 or 4
// in flight per thread).  Before every launch a 512 MB read-only pass
// replaces the 256 MB memory-side cache's contents with clean lines, so no
// timed pass starts with its own data cached or with dirty lines to write
// back.  Two warm-ups and five timed launches per pass (HIP events); prints
// one JSON line with the best and median rate of each pass.
// Standalone measurement tool built in-tree beside the library; it shares no
// code with it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kThreads = 256;

template <int U, bool NT>
__global__ __launch_bounds__(kThreads) void read_pass(const u32x4* __restrict__ s, size_t n,
                                                      uint32_t* __restrict__ out) {
  const size_t base = (size_t)blockIdx.x * kThreads * U + threadIdx.x;
  u32x4 w[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const size_t i = base + (size_t)u * kThreads;
    w[u] = i < n ? (NT ? __builtin_nontemporal_load(s + i) : s[i]) : (u32x4)0;
  }
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) x ^= w[u][0] ^ w[u][1] ^ w[u][2] ^ w[u][3];
  if (x == 0x9E3779B9u) out[blockIdx.x] = x;
}

template <int U, bool NT>
__global__ __launch_bounds__(kThreads) void copy_pass(const u32x4* __restrict__ s, u32x4* __restrict__ d, size_t n) {
  const size_t base = (size_t)blockIdx.x * kThreads * U + threadIdx.x;
  u32x4 w[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const size_t i = base + (size_t)u * kThreads;
    if (i < n) w[u] = NT ? __builtin_nontemporal_load(s + i) : s[i];
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const size_t i = base + (size_t)u * kThreads;
    if (i < n) d[i] = w[u];
  }
}

template <int U>
__global__ __launch_bounds__(kThreads) void write_pass(u32x4* __restrict__ d, size_t n) {
  const size_t base = (size_t)blockIdx.x * kThreads * U + threadIdx.x;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const size_t i = base + (size_t)u * kThreads;
    if (i < n) d[i] = (u32x4){(uint32_t)i, 1u, 2u, 3u};
  }
}

struct Bufs {
  u32x4 *a = nullptr, *b = nullptr, *flush = nullptr;
  uint32_t* out = nullptr;
  size_t n = 0, nw = 0, nflush = 0;
};

bool ok(hipError_t e) { return e == hipSuccess; }

template <typename F>
bool time_pass(const Bufs& m, F launch, double bytes, double& best, double& median) {
  hipEvent_t e0, e1;
  if (!ok(hipEventCreate(&e0)) || !ok(hipEventCreate(&e1))) return false;
  std::vector<double> rates;
  for (int rep = 0; rep < 7; ++rep) {
    hipLaunchKernelGGL((read_pass<4, false>), dim3((unsigned)((m.nflush + kThreads * 4 - 1) / (kThreads * 4))),
                       dim3(kThreads), 0, 0, m.flush, m.nflush, m.out);
    if (!ok(hipEventRecord(e0))) return false;
    launch();
    if (!ok(hipEventRecord(e1)) || !ok(hipEventSynchronize(e1))) return false;
    float ms = 0.0f;
    if (!ok(hipEventElapsedTime(&ms, e0, e1))) return false;
    if (rep >= 2) rates.push_back(bytes / (ms * 1e-3) / 1e9);
  }
  std::sort(rates.begin(), rates.end());
  best = rates.back();
  median = rates[rates.size() / 2];
  return ok(hipEventDestroy(e0)) && ok(hipEventDestroy(e1));
}

unsigned grid(size_t n, int u) { return (unsigned)((n + (size_t)kThreads * u - 1) / ((size_t)kThreads * u)); }

template <int U, bool NT>
bool run_kind(const Bufs& m, int kind, double bytes, double& best, double& med) {
  if (kind == 0)
    return time_pass(m, [&] { hipLaunchKernelGGL((read_pass<U, NT>), dim3(grid(m.n, U)), dim3(kThreads), 0, 0,
                                                  m.a, m.n, m.out); }, bytes, best, med);
  if (kind == 1)
    return time_pass(m, [&] { hipLaunchKernelGGL((copy_pass<U, NT>), dim3(grid(m.n, U)), dim3(kThreads), 0, 0,
                                                  m.a, m.b, m.n); }, bytes, best, med);
  return time_pass(m, [&] { hipLaunchKernelGGL((write_pass<U>), dim3(grid(m.nw, U)), dim3(kThreads), 0, 0,
                                                m.b, m.nw); }, bytes, best, med);
}

bool run_pass(const Bufs& m, int kind, int u, bool nt, double bytes, double& best, double& med) {
  if (u == 1) return nt ? run_kind<1, true>(m, kind, bytes, best, med) : run_kind<1, false>(m, kind, bytes, best, med);
  return nt ? run_kind<4, true>(m, kind, bytes, best, med) : run_kind<4, false>(m, kind, bytes, best, med);
}

}  // namespace

int main() {
  Bufs m;
  m.n = (size_t)40 * 109000 * 128 * 2 / 16;          // one BF16 input tensor, in 16-byte vectors
  m.nw = (size_t)40 * 109000 * (64 + 8) / 16;         // its codes and scales
  m.nflush = ((size_t)512 << 20) / 16;
  if (!ok(hipMalloc(&m.a, m.n * 16)) || !ok(hipMalloc(&m.b, m.n * 16)) || !ok(hipMalloc(&m.flush, m.nflush * 16)) ||
      !ok(hipMalloc(&m.out, (size_t)grid(m.n, 1) * 4)) || !ok(hipMemset(m.a, 0x3C, m.n * 16)) ||
      !ok(hipMemset(m.b, 0, m.n * 16)) || !ok(hipMemset(m.flush, 0x11, m.nflush * 16)) ||
      !ok(hipDeviceSynchronize())) {
    fprintf(stderr, "hbm_ceiling_probe: allocation failed\n");
    return 1;
  }
  struct Pass {
    const char* name;
    int kind;        // 0 read, 1 copy, 2 write
    int u;
    bool nt;
  };
  const Pass passes[] = {{"read_u1", 0, 1, false},    {"read_u4", 0, 4, false}, {"read_nt_u1", 0, 1, true},
                         {"read_nt_u4", 0, 4, true},  {"copy_u1", 1, 1, false}, {"copy_u4", 1, 4, false},
                         {"copy_nt_u1", 1, 1, true},  {"copy_nt_u4", 1, 4, true}, {"write_u1", 2, 1, false},
                         {"write_u4", 2, 4, false}};
  std::string js = "{\"hbm_ceiling_GB/s\": {";
  bool first = true;
  for (const Pass& p : passes) {
    double best = 0.0, med = 0.0;
    const double bytes = p.kind == 0 ? (double)m.n * 16 : p.kind == 1 ? 2.0 * (double)m.n * 16 : (double)m.nw * 16;
    if (!run_pass(m, p.kind, p.u, p.nt, bytes, best, med)) {
      fprintf(stderr, "hbm_ceiling_probe: %s failed\n", p.name);
      return 1;
    }
    char buf[160];
    snprintf(buf, sizeof buf, "%s\"%s\": {\"bytes\": %.0f, \"best\": %.1f, \"median\": %.1f}", first ? "" : ", ",
             p.name, bytes, best, med);
    js += buf;
    first = false;
  }
  js += "}, \"tensor\": \"[40, 109000, 128] bf16\"}";
  if (!ok(hipDeviceSynchronize())) return 1;
  printf("%s\n", js.c_str());
  return 0;
}
