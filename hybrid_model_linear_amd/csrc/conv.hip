// Short causal depthwise conv1d (width K, bf16) with SiLU, the step that produces
// mixed_qkv in front of the GDN layer, over packed sequences, with each sequence's
// last K - 1 inputs kept per slot in a conv-state pool (the conv[0] buffer next to
// the temporal state in the hybrid model's memory pool: SGLang GDN test-matrix
// article, memory-pool section).
//
// HBM-bound (2 bytes in and 2 out per channel and token against 2K flops): a thread
// owns 8 adjacent channels, one 16-byte vector of a token row, and walks a tile of
// tokens with the K - 1 previous inputs in registers, so x is read once and out
// written once; a tile re-reads only the K - 1 rows before it (from L2).  The
// window restarts from the pool at every sequence start inside a tile.  The new
// states are written by a second launch, so that no workgroup rewrites a slot that
// another one has still to read.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kCV = 8;           // channels per thread (one 16-byte bf16 vector)
constexpr int kCThreads = 128;   // threads per workgroup: 1024 channels
constexpr int kCTok = 64;        // tokens per workgroup of the output pass
constexpr int kCAhead = 8;       // token rows loaded ahead of their use

struct V8 {
  float f[kCV];
};

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
// Outputs and states are streamed out with non-temporal stores: nothing in the kernel
// reads them again, and keeping them out of L2 leaves it to the rows the next tile
// re-reads (about 10% faster than plain stores at 8 x 4096 x 8192).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st16(uint16_t* p, uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}

__device__ __forceinline__ V8 unpack(uint4 u) {
  V8 r;
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.f[2 * i] = __uint_as_float(w[i] << 16);
    r.f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
  return r;
}

__device__ __forceinline__ uint4 pack(const V8& v) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)f32_to_bf16(v.f[2 * i]) | ((uint32_t)f32_to_bf16(v.f[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// M values per channel for 8 channels, stored channel-major (a channel's M values
// contiguous): 8 M bf16 = M 16-byte vectors.  v[j][c] = value j of channel c.  Used
// for the taps (M = K) and the conv state (M = K - 1); bf16 values round-trip exactly.
template <int M>
struct Block8 {
  float v[M][kCV];
  __device__ __forceinline__ void load(const uint16_t* p) {
    uint32_t w[4 * M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const uint4 u = ld16(p + 8 * i);
      w[4 * i] = u.x;
      w[4 * i + 1] = u.y;
      w[4 * i + 2] = u.z;
      w[4 * i + 3] = u.w;
    }
#pragma unroll
    for (int c = 0; c < kCV; ++c)
#pragma unroll
      for (int j = 0; j < M; ++j) {
        const int e = c * M + j;
        v[j][c] = __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
      }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int j = 0; j < M; ++j)
#pragma unroll
      for (int c = 0; c < kCV; ++c) v[j][c] = 0.0f;
  }
  __device__ __forceinline__ void store(uint16_t* p) const {
    uint32_t w[4 * M];
#pragma unroll
    for (int i = 0; i < 4 * M; ++i) w[i] = 0;
#pragma unroll
    for (int c = 0; c < kCV; ++c)
#pragma unroll
      for (int j = 0; j < M; ++j) {
        const int e = c * M + j;
        const uint32_t h = f32_to_bf16(v[j][c]);
        w[e >> 1] |= (e & 1) ? (h << 16) : h;
      }
#pragma unroll
    for (int i = 0; i < M; ++i)
      st16(p + 8 * i, make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]));
  }
};

// One output row of 8 channels: bias + sum_j tap_j * window_j (window K - 1 past
// inputs, oldest first, then the current input), then silu.  silu(y) = y / (1 + e^-y)
// with the hardware exp and reciprocal (a few ulp, far below the bf16 rounding).
template <int K, bool kAct>
__device__ __forceinline__ uint4 conv_row(const Block8<K>& tap, const float (&bias)[kCV],
                                          const float (&win)[K - 1][kCV], const V8& x) {
  V8 y;
#pragma unroll
  for (int c = 0; c < kCV; ++c) {
    float acc = bias[c];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) acc = fmaf(tap.v[j][c], win[j][c], acc);
    acc = fmaf(tap.v[K - 1][c], x.f[c], acc);
    if constexpr (kAct) acc = acc * __builtin_amdgcn_rcpf(1.0f + __expf(-acc));
    y.f[c] = acc;
  }
  return pack(y);
}

template <int K>
__device__ __forceinline__ void load_taps(const ConvLaunch& p, int c0, Block8<K>& tap, float (&bias)[kCV]) {
  tap.load(p.weight + (int64_t)c0 * K);
  // branch-free, so that the loads issue together: without a bias, read 8 in-bounds
  // taps (c0 + 8 <= D <= D K) and select zero
  const bool has_bias = p.bias != nullptr;
  const V8 b = unpack(ld16((has_bias ? p.bias : p.weight) + c0));
#pragma unroll
  for (int c = 0; c < kCV; ++c) bias[c] = has_bias ? b.f[c] : 0.0f;
}

// ------------------------------------------------------------------ varlen outputs
// Workgroup (token tile, 1024-channel block).  The token-to-sequence walk depends only
// on the tile, so every branch on it is uniform.
template <int K, bool kAct>
__global__ void __launch_bounds__(kCThreads) conv_out_kernel(const ConvLaunch p) {
  const int c0 = (blockIdx.y * kCThreads + threadIdx.x) * kCV;
  if (c0 >= p.D) return;
  const int64_t t0 = (int64_t)blockIdx.x * kCTok;
  const int64_t tend = t0 + kCTok < p.T ? t0 + kCTok : p.T;
  if (t0 >= p.cu[p.N]) return;     // tokens past the last sequence are padding

  Block8<K> tap;
  float bias[kCV];
  load_taps<K>(p, c0, tap, bias);

  // the sequence holding t0: the last n with cu[n] <= t0 (skips empty ones)
  int lo = 0, hi = p.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.cu[mid] <= t0) lo = mid; else hi = mid - 1;
  }
  int n = lo;
  int64_t s0 = p.cu[n], nb = p.cu[n + 1];
  bool live = p.slot[n] >= 0;

  // window of token t of sequence n: entry j is input i - (K - 1) + j of the
  // sequence (i = t - s0), a negative index being an entry of the slot's old state
  float win[K - 1][kCV];
  auto start = [&](int64_t t) __attribute__((always_inline)) {
    const int64_t i = t - s0;
    const int s = p.slot[n];
    Block8<K - 1> st;
    if (i < K - 1 && s >= 0 && (!p.has_init || p.has_init[n] != 0))
      st.load(p.pool + (int64_t)s * p.pool_stride + (int64_t)c0 * (K - 1));
    else
      st.zero();
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
      const int64_t r = i - (K - 1) + j;
      if (r >= 0) {
        const V8 v = unpack(ld16(p.x + (s0 + r) * p.x_stride + c0));
#pragma unroll
        for (int c = 0; c < kCV; ++c) win[j][c] = v.f[c];
      } else {
#pragma unroll
        for (int e = 0; e < K - 1; ++e)   // state entry r + K - 1, selected without indexing
          if (e == r + K - 1) {
#pragma unroll
            for (int c = 0; c < kCV; ++c) win[j][c] = st.v[e][c];
          }
      }
    }
  };
  start(t0);

  for (int64_t tb = t0; tb < tend; tb += kCAhead) {
    // all rows of the batch loaded at once (a row past the end reads the last row
    // again, in bounds and unused), so that no load waits for the one before it
    uint4 xr[kCAhead];
#pragma unroll
    for (int u = 0; u < kCAhead; ++u)
      xr[u] = ld16(p.x + (tb + u < tend ? tb + u : tend - 1) * p.x_stride + c0);
#pragma unroll
    for (int u = 0; u < kCAhead; ++u) {
      const int64_t t = tb + u;
      if (t >= tend) break;
      if (t == nb) {               // sequence n ends before t
        while (n + 1 < p.N && p.cu[n + 2] <= t) ++n;   // skip empty ones
        if (n + 1 >= p.N) {        // past the last sequence: padding, nothing written
          tb = tend;
          break;
        }
        ++n;                       // the sequence starting at t
        s0 = t;
        nb = p.cu[n + 1];
        live = p.slot[n] >= 0;
        start(t);
      }
      const V8 xv = unpack(xr[u]);
      if (live) st16(p.out + t * p.out_stride + c0, conv_row<K, kAct>(tap, bias, win, xv));
#pragma unroll
      for (int j = 0; j + 1 < K - 1; ++j)
#pragma unroll
        for (int c = 0; c < kCV; ++c) win[j][c] = win[j + 1][c];
#pragma unroll
      for (int c = 0; c < kCV; ++c) win[K - 2][c] = xv.f[c];
    }
  }
}

// ------------------------------------------------------------------ token trees
// Target verify with a token tree: workgroup (token, 1024-channel block).  The window
// follows the token's parents back to the sequence start and then the slot's state;
// a few tokens per sequence, so each token walks its own path (K - 1 parent reads).
template <int K, bool kAct>
__global__ void __launch_bounds__(kCThreads) conv_tree_kernel(const ConvLaunch p) {
  const int c0 = (blockIdx.y * kCThreads + threadIdx.x) * kCV;
  if (c0 >= p.D) return;
  const int64_t t = blockIdx.x;
  int lo = 0, hi = p.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int n = lo;
  const int s = p.slot[n];
  if (s < 0 || t >= p.cu[n + 1]) return;    // skipped sequence, or padding past the last
  const int64_t s0 = p.cu[n];
  Block8<K> tap;
  float bias[kCV];
  load_taps<K>(p, c0, tap, bias);
  const V8 xv = unpack(ld16(p.x + t * p.x_stride + c0));
  // rows of the K - 1 inputs before t on its root path, newest first; -1 once the
  // path has passed the start (a parent outside [0, index) ends the path there)
  int64_t row[K - 1];
  int64_t cur = t - s0;
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    if (cur >= 0) {
      const int64_t par = p.parent[s0 + cur];
      cur = (par >= 0 && par < cur) ? par : -1;
    }
    row[j] = cur >= 0 ? s0 + cur : -1;
  }
  Block8<K - 1> st;
  if (row[K - 2] < 0 && (!p.has_init || p.has_init[n] != 0))
    st.load(p.pool + (int64_t)s * p.pool_stride + (int64_t)c0 * (K - 1));
  else
    st.zero();
  // window oldest first: entry K - 2 - j is path input j; past the start, path input
  // j is state entry K - 2 - m for the m-th step beyond it
  float win[K - 1][kCV];
  int m = 0;
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    if (row[j] >= 0) {
      const V8 v = unpack(ld16(p.x + row[j] * p.x_stride + c0));
#pragma unroll
      for (int c = 0; c < kCV; ++c) win[K - 2 - j][c] = v.f[c];
    } else {
#pragma unroll
      for (int e = 0; e < K - 1; ++e)
        if (e == K - 2 - m) {
#pragma unroll
          for (int c = 0; c < kCV; ++c) win[K - 2 - j][c] = st.v[e][c];
        }
      ++m;
    }
  }
  st16(p.out + t * p.out_stride + c0, conv_row<K, kAct>(tap, bias, win, xv));
}

// ------------------------------------------------------------------ varlen states
// Workgroup (sequence, 1024-channel block): the last K - 1 window entries of the
// sequence, partly its old state when it is shorter than K - 1.
template <int K>
__global__ void __launch_bounds__(kCThreads) conv_state_kernel(const ConvLaunch p) {
  const int c0 = (blockIdx.y * kCThreads + threadIdx.x) * kCV;
  if (c0 >= p.D) return;
  const int n = blockIdx.x;
  const int s = p.slot[n];
  if (s < 0) return;
  const int64_t s0 = p.cu[n];
  const int64_t len = p.cu[n + 1] - s0;
  uint16_t* dst = p.pool + (int64_t)s * p.pool_stride + (int64_t)c0 * (K - 1);
  Block8<K - 1> old, nw;
  if (len < K - 1 && (!p.has_init || p.has_init[n] != 0))
    old.load(dst);
  else
    old.zero();
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    const int64_t r = len - (K - 1) + j;
    if (r >= 0) {
      const V8 v = unpack(ld16(p.x + (s0 + r) * p.x_stride + c0));
#pragma unroll
      for (int c = 0; c < kCV; ++c) nw.v[j][c] = v.f[c];
    } else {
#pragma unroll
      for (int e = 0; e < K - 1; ++e)
        if (e == r + K - 1) {
#pragma unroll
          for (int c = 0; c < kCV; ++c) nw.v[j][c] = old.v[e][c];
        }
    }
  }
  nw.store(dst);
}

// ------------------------------------------------------------------ decode
// Workgroup (row, 1024-channel block): one token from the slot's state, and the
// state shifted by one.  Each (row, channel) is read and written by one thread, so
// out may be x itself.
template <int K, bool kAct>
__global__ void __launch_bounds__(kCThreads) conv_update_kernel(const ConvLaunch p) {
  const int c0 = (blockIdx.y * kCThreads + threadIdx.x) * kCV;
  if (c0 >= p.D) return;
  const int b = blockIdx.x;
  // x and the taps do not depend on the slot: issue them before its check
  const V8 xv = unpack(ld16(p.x + (int64_t)b * p.x_stride + c0));
  Block8<K> tap;
  float bias[kCV];
  load_taps<K>(p, c0, tap, bias);
  const int s = p.slot[b];
  if (s < 0) return;
  uint16_t* sp = p.pool + (int64_t)s * p.pool_stride + (int64_t)c0 * (K - 1);
  Block8<K - 1> st;
  st.load(sp);
  st16(p.out + (int64_t)b * p.out_stride + c0, conv_row<K, kAct>(tap, bias, st.v, xv));
  if (p.keep_pool) return;
#pragma unroll
  for (int j = 0; j + 1 < K - 1; ++j)
#pragma unroll
    for (int c = 0; c < kCV; ++c) st.v[j][c] = st.v[j + 1][c];
#pragma unroll
  for (int c = 0; c < kCV; ++c) st.v[K - 2][c] = xv.f[c];
  st.store(sp);
}

template <int K>
hipError_t launch_k(const ConvLaunch& p, bool update, hipStream_t stream) {
  const unsigned cblocks = (unsigned)((p.D / kCV + kCThreads - 1) / kCThreads);
  if (update) {
    if (p.N > 0) {
      const dim3 grid((unsigned)p.N, cblocks);
      if (p.act) hipLaunchKernelGGL((conv_update_kernel<K, true>), grid, dim3(kCThreads), 0, stream, p);
      else hipLaunchKernelGGL((conv_update_kernel<K, false>), grid, dim3(kCThreads), 0, stream, p);
    }
    return hipGetLastError();
  }
  if (p.parent) {   // token tree: per-token windows, the pool only read
    if (p.T > 0) {
      const dim3 grid((unsigned)p.T, cblocks);
      if (p.act) hipLaunchKernelGGL((conv_tree_kernel<K, true>), grid, dim3(kCThreads), 0, stream, p);
      else hipLaunchKernelGGL((conv_tree_kernel<K, false>), grid, dim3(kCThreads), 0, stream, p);
    }
    return hipGetLastError();
  }
  if (p.T > 0) {
    const dim3 grid((unsigned)((p.T + kCTok - 1) / kCTok), cblocks);
    if (p.act) hipLaunchKernelGGL((conv_out_kernel<K, true>), grid, dim3(kCThreads), 0, stream, p);
    else hipLaunchKernelGGL((conv_out_kernel<K, false>), grid, dim3(kCThreads), 0, stream, p);
  }
  if (!p.keep_pool && p.N > 0)
    hipLaunchKernelGGL((conv_state_kernel<K>), dim3((unsigned)p.N, cblocks), dim3(kCThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_any(const ConvLaunch& p, bool update, hipStream_t stream) {
  switch (p.K) {
    case 2: return launch_k<2>(p, update, stream);
    case 3: return launch_k<3>(p, update, stream);
    case 4: return launch_k<4>(p, update, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_conv(const ConvLaunch& p, hipStream_t stream) { return launch_any(p, false, stream); }
hipError_t launch_conv_update(const ConvLaunch& p, hipStream_t stream) { return launch_any(p, true, stream); }

}  // namespace gdn
