// Bandwidth probes for the benchmark (not part of libmhc): plain streaming
// kernels that read, write or copy a device buffer once, giving the HBM
// rates this device actually reaches for each access mix.  The benchmark
// reports the mHC kernels' achieved bandwidth as a fraction of these.
//
// Layout for MI355X: 16-byte vectors per lane (1 KiB per wave instruction),
// four independent vectors in flight per lane per loop trip, non-temporal
// loads and stores (the data is touched once), a grid of 8 workgroups of 256
// lanes per compute unit walking the buffer in grid-sized strides.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4 *__restrict__ src, int64_t nv,
                                                        uint32_t *__restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < nv; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < nv; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  // Keeps the loads live; a value of 0x5EED is never expected, so this store
  // practically never happens.
  if (acc == 0x5EEDu) sink[0] = acc;
}

__global__ __launch_bounds__(kThreads) void write_kernel(u32x4 *__restrict__ dst, int64_t nv, uint32_t val) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const u32x4 v = {val, val, val, val};
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nv; i += stride)
    __builtin_nontemporal_store(v, dst + i);
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                        int64_t nv) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < nv; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < nv; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Tiled variants: every wave owns kRun consecutive KiB (64 lanes x 16 B per
// instruction), all issued before any is used; one wave per workgroup and
// one workgroup per run, so the dispatcher walks the buffer in order (the
// pattern of the library's streaming kernels).  NT selects non-temporal
// stores.
constexpr int kRun = 4;
__global__ __launch_bounds__(64) void read_tiled(const u32x4 *__restrict__ src, int64_t nv,
                                                 uint32_t *__restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * 64 * kRun + threadIdx.x;
  uint32_t acc = 0;
  u32x4 v[kRun];
#pragma unroll
  for (int u = 0; u < kRun; ++u) v[u] = base + 64 * u < nv ? __builtin_nontemporal_load(src + base + 64 * u) : u32x4{};
#pragma unroll
  for (int u = 0; u < kRun; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  if (acc == 0x5EEDu) sink[0] = acc;
}
template <bool NT>
__global__ __launch_bounds__(64) void write_tiled(u32x4 *__restrict__ dst, int64_t nv, uint32_t val) {
  const int64_t base = (int64_t)blockIdx.x * 64 * kRun + threadIdx.x;
  const u32x4 v = {val, val, val, val};
#pragma unroll
  for (int u = 0; u < kRun; ++u)
    if (base + 64 * u < nv) {
      if constexpr (NT) __builtin_nontemporal_store(v, dst + base + 64 * u);
      else dst[base + 64 * u] = v;
    }
}
template <bool NT>
__global__ __launch_bounds__(64) void copy_tiled(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, int64_t nv) {
  const int64_t base = (int64_t)blockIdx.x * 64 * kRun + threadIdx.x;
  u32x4 v[kRun];
#pragma unroll
  for (int u = 0; u < kRun; ++u) v[u] = base + 64 * u < nv ? __builtin_nontemporal_load(src + base + 64 * u) : u32x4{};
#pragma unroll
  for (int u = 0; u < kRun; ++u)
    if (base + 64 * u < nv) {
      if constexpr (NT) __builtin_nontemporal_store(v[u], dst + base + 64 * u);
      else dst[base + 64 * u] = v[u];
    }
}

int grid_for(int64_t nv) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t want = (int64_t)cus * 8;
  const int64_t need = (nv + kThreads - 1) / kThreads;
  return (int)(need < want ? (need > 0 ? need : 1) : want);
}

}  // namespace

extern "C" {

// mode 0: read `bytes` of src; 1: write `bytes` of dst; 2: copy src -> dst;
// plus 16 * variant: 0 the grid-stride kernels (8 workgroups of 256 lanes per
// CU), 1 the tiled kernels with non-temporal stores, 2 the tiled kernels with
// plain stores.  bytes must be a multiple of 16 and the pointers 16-byte
// aligned; sink is a 4-byte device word (read mode only).  Returns a
// hipError_t value.
int mhc_probe_bandwidth(int mode, const void *src, void *dst, int64_t bytes, void *sink, void *stream) {
  if (bytes <= 0 || bytes % 16 != 0) return (int)hipErrorInvalidValue;
  const int64_t nv = bytes / 16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int variant = mode >> 4;
  mode &= 15;
  if (variant == 1 || variant == 2) {
    const int64_t blocks = (nv + 64 * kRun - 1) / (64 * kRun);
    if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
    const dim3 grid((uint32_t)blocks);
    const u32x4 *s = static_cast<const u32x4 *>(src);
    u32x4 *d = static_cast<u32x4 *>(dst);
    switch (mode) {
      case 0: read_tiled<<<grid, 64, 0, st>>>(s, nv, static_cast<uint32_t *>(sink)); break;
      case 1:
        if (variant == 1) write_tiled<true><<<grid, 64, 0, st>>>(d, nv, 0x3F803F80u);
        else write_tiled<false><<<grid, 64, 0, st>>>(d, nv, 0x3F803F80u);
        break;
      case 2:
        if (variant == 1) copy_tiled<true><<<grid, 64, 0, st>>>(s, d, nv);
        else copy_tiled<false><<<grid, 64, 0, st>>>(s, d, nv);
        break;
      default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
  }
  if (variant != 0) return (int)hipErrorInvalidValue;
  const int g = grid_for(nv);
  switch (mode) {
    case 0:
      read_kernel<<<g, kThreads, 0, st>>>(static_cast<const u32x4 *>(src), nv, static_cast<uint32_t *>(sink));
      break;
    case 1: write_kernel<<<g, kThreads, 0, st>>>(static_cast<u32x4 *>(dst), nv, 0x3F803F80u); break;
    case 2:
      copy_kernel<<<g, kThreads, 0, st>>>(static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), nv);
      break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // extern "C"
