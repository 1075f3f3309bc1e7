// Backward of the proxy-compensated route (the PrimTS page, "proxy-compensated
// block-sparse attention", flashinfer pull request 4872: description, proxy
// paragraph; the backward is the derivative of that forward).
//
// By its definition the route is attention over keys rebuilt token by token:
// a Q block's listed blocks with their own tokens, and every other block n as
// c_n copies of (mean key, summed value / c_n), c_n its token count.  The c_n
// copies of one key are one key whose exponential is weighted by c_n, i.e.
// with log c_n added to its score, so the backward runs the block-sparse
// backward kernels on an extended KV sequence: the N blocks of keys and
// values, then one key per block holding its summaries (mean key, summed
// value / c_n), in chunks of block_kv summaries.  A Q block lists the blocks
// it attends exactly and the chunks holding summaries it takes; a per-row
// bit set says which summaries of a chunk those are, and the kernels add
// log2 c_n to a summary's exponent.  The score of a summary key has the
// gradient of the c_n copies' scores summed, so d(mean key) is the summary
// key's dK, and d(summed value) its dV over c_n (the kernels write both).
// The kernels here build the extended K/V and the extended block mask and
// bit sets (HBM-bound, a few hundred MB on the page's workload).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsa_fwd_common.h"

namespace bsa {
namespace {

using namespace dev;

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Extended K/V, contiguous [B, (N + Nc)*bk, Hkv, D]: rows t < N*bk are K and V
// (zero past Sk), row N*bk + u the summaries at position u (block u for
// u < nreg, the last block at lastpos), the summed value divided by c_n and
// rounded to bf16; zero elsewhere.  A thread moves 8 head_dim elements (16
// bytes) of one row.
__global__ __launch_bounds__(256) void proxy_expand_kernel(ProxyBwdParams p, int64_t chunks) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= chunks) return;
  const int cpr = p.D / 8;
  const int64_t row = c / cpr;
  const int d0 = (int)(c % cpr) * 8;
  const int hk = (int)(row % p.Hkv);
  const int64_t bt = row / p.Hkv;
  const int64_t Sx = (int64_t)(p.N + p.Nc) * p.bk;
  const int t = (int)(bt % Sx), b = (int)(bt / Sx);
  uint4 kw = make_uint4(0, 0, 0, 0), vw = make_uint4(0, 0, 0, 0);
  const int half = p.N * p.bk;
  const int u = t - half;
  const int n = u < p.nreg ? u : (u == p.lastpos ? p.N - 1 : -1);
  if (t < half) {
    if (t < p.Sk) {
      kw = *reinterpret_cast<const uint4*>(p.k + b * p.k_sb + (int64_t)t * p.k_ss + hk * p.k_sh + d0);
      vw = *reinterpret_cast<const uint4*>(p.v + b * p.v_sb + (int64_t)t * p.v_ss + hk * p.v_sh + d0);
    }
  } else if (n >= 0) {
    const int cn = min(p.bk, p.Sk - n * p.bk);
    kw = *reinterpret_cast<const uint4*>(p.ks + b * p.ks_sb + (int64_t)n * p.ks_sn + hk * p.ks_sh + d0);
    const uint4 s = *reinterpret_cast<const uint4*>(p.vs + b * p.vs_sb + (int64_t)n * p.vs_sn +
                                                     hk * p.vs_sh + d0);
    const float inv = 1.f / (float)cn;
    vw = make_uint4(pack_bf16x2(bf_lo(s.x) * inv, bf_hi(s.x) * inv),
                    pack_bf16x2(bf_lo(s.y) * inv, bf_hi(s.y) * inv),
                    pack_bf16x2(bf_lo(s.z) * inv, bf_hi(s.z) * inv),
                    pack_bf16x2(bf_lo(s.w) * inv, bf_hi(s.w) * inv));
  }
  const int64_t o = row * p.D + d0;
  *reinterpret_cast<uint4*>(p.kx + o) = kw;
  *reinterpret_cast<uint4*>(p.vx + o) = vw;
}

// One workgroup (four waves) per Q-block row (b, h, i): marks the blocks the
// row lists (either list; ids outside [0, N) skipped) in maskx[0 .. N), then
// the bit set of the summary positions it takes (those of the blocks it does
// not list), one word of 64 per ballot, and maskx[N + g] for the chunks
// holding any of them.
__global__ __launch_bounds__(256) void proxy_ext_mask_kernel(ProxyBwdParams p) {
  const int rowid = blockIdx.x;
  const int i = rowid % p.M, bh = rowid / p.M;
  const int h = bh % p.H, b = bh / p.H;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint8_t* row = p.maskx + (int64_t)rowid * (p.N + p.Nc);
  uint64_t* words = p.keep + (int64_t)rowid * p.W;
  for (int n = threadIdx.x; n < p.N; n += blockDim.x) row[n] = 0;
  __syncthreads();
  for (int list = 0; list < 2; ++list) {
    const int32_t* cnt = list == 0 ? p.mcnt : p.fcnt;
    if (cnt == nullptr) continue;
    const int64_t* cs = list == 0 ? p.mc_s : p.fc_s;
    const int64_t* is = list == 0 ? p.mi_s : p.fi_s;
    const int32_t* idx = (list == 0 ? p.midx : p.fidx) + b * is[0] + h * is[1] + i * is[2];
    const int c = min(max(cnt[b * cs[0] + h * cs[1] + i * cs[2]], 0), p.N);
    for (int e = threadIdx.x; e < c; e += blockDim.x) {
      const int j = idx[(int64_t)e * is[3]];
      if (j >= 0 && j < p.N) row[j] = 1;
    }
  }
  __syncthreads();
  // position u holds block u (u < nreg) or the last block (u == lastpos)
  auto taken = [&](int u) {
    const int n = u < p.nreg ? u : (u == p.lastpos ? p.N - 1 : -1);
    return n >= 0 && row[n] == 0;
  };
  for (int wi = wv; wi < p.W; wi += blockDim.x / 64) {
    const uint64_t bits = __ballot(taken(64 * wi + lane));
    if (lane == 0) words[wi] = bits;
  }
  for (int g = threadIdx.x; g < p.Nc; g += blockDim.x) {
    bool any = false;
    for (int u = g * p.bk; u < (g + 1) * p.bk && !any; ++u) any = taken(u);
    row[p.N + g] = any;
  }
}

}  // namespace

hipError_t launch_proxy_bwd_prepare(const ProxyBwdParams& p, hipStream_t s) {
  const int64_t chunks = (int64_t)p.B * (p.N + p.Nc) * p.bk * p.Hkv * (p.D / 8);
  if (chunks > 0)
    hipLaunchKernelGGL(proxy_expand_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0,
                       s, p, chunks);
  const int64_t rows = (int64_t)p.B * p.H * p.M;
  if (rows > 0)
    hipLaunchKernelGGL(proxy_ext_mask_kernel, dim3((unsigned)rows), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace bsa
