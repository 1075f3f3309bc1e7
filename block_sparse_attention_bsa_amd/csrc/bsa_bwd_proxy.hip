// Backward of the proxy-compensated route (the PrimTS page, "proxy-compensated
// block-sparse attention", flashinfer pull request 4872: description, proxy
// paragraph; the backward is the derivative of that forward).
//
// By its definition the route is attention over keys rebuilt token by token:
// a Q block's listed blocks with their own tokens, and every other block n as
// c_n copies of (mean key, summed value / c_n), c_n its token count.  The
// backward therefore runs the block-sparse backward kernels on an extended
// KV sequence of 2N blocks of block_kv rows: blocks 0..N-1 hold K and V,
// blocks N..2N-1 hold the copies of the summaries.  Each Q block lists the
// blocks it attends exactly and the copies of the blocks it omits; the
// valid-count mask_mod keeps c_n rows of each.  The gradients of the copies
// give those of the summaries: each copy of block n gets the same gradient,
// so d(mean key) is c_n times a copy's dK and d(summed value) is a copy's dV.
// The kernels here are the three HBM-bound steps around that backward:
// building the extended K/V, the extended block mask and valid counts, and
// reading the gradients back out.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsa_fwd_common.h"

namespace bsa {
namespace {

using namespace dev;

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Extended K/V, contiguous [B, 2*N*bk, Hkv, D]: rows t < N*bk are K and V (zero
// past Sk), rows N*bk + n*bk + r are, for r < c_n, the mean key of block n and
// its summed value divided by c_n (rounded to bf16), else zero.  A thread
// moves 8 head_dim elements (16 bytes) of one row.
__global__ __launch_bounds__(256) void proxy_expand_kernel(ProxyBwdParams p, int64_t chunks) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= chunks) return;
  const int cpr = p.D / 8;
  const int64_t row = c / cpr;
  const int d0 = (int)(c % cpr) * 8;
  const int hk = (int)(row % p.Hkv);
  const int64_t bt = row / p.Hkv;
  const int64_t Sx = 2 * (int64_t)p.N * p.bk;
  const int t = (int)(bt % Sx), b = (int)(bt / Sx);
  uint4 kw = make_uint4(0, 0, 0, 0), vw = make_uint4(0, 0, 0, 0);
  const int half = p.N * p.bk;
  if (t < half) {
    if (t < p.Sk) {
      kw = *reinterpret_cast<const uint4*>(p.k + b * p.k_sb + (int64_t)t * p.k_ss + hk * p.k_sh + d0);
      vw = *reinterpret_cast<const uint4*>(p.v + b * p.v_sb + (int64_t)t * p.v_ss + hk * p.v_sh + d0);
    }
  } else {
    const int n = (t - half) / p.bk, r = (t - half) % p.bk;
    const int cn = min(p.bk, p.Sk - n * p.bk);
    if (r < cn) {
      kw = *reinterpret_cast<const uint4*>(p.ks + b * p.ks_sb + (int64_t)n * p.ks_sn + hk * p.ks_sh + d0);
      const uint4 s = *reinterpret_cast<const uint4*>(p.vs + b * p.vs_sb + (int64_t)n * p.vs_sn +
                                                       hk * p.vs_sh + d0);
      const float inv = 1.f / (float)cn;
      vw = make_uint4(pack_bf16x2(bf_lo(s.x) * inv, bf_hi(s.x) * inv),
                      pack_bf16x2(bf_lo(s.y) * inv, bf_hi(s.y) * inv),
                      pack_bf16x2(bf_lo(s.z) * inv, bf_hi(s.z) * inv),
                      pack_bf16x2(bf_lo(s.w) * inv, bf_hi(s.w) * inv));
    }
  }
  const int64_t o = row * p.D + d0;
  *reinterpret_cast<uint4*>(p.kx + o) = kw;
  *reinterpret_cast<uint4*>(p.vx + o) = vw;
}

// Extended block mask [B, H, M, 2N] (one workgroup per Q-block row): block n
// when the row lists it (either list), block N + n when it does not; and the
// valid counts [2N] (c_n for both).  Ids outside [0, N) are skipped.
__global__ __launch_bounds__(256) void proxy_ext_mask_kernel(ProxyBwdParams p) {
  const int rowid = blockIdx.x;
  const int i = rowid % p.M, bh = rowid / p.M;
  const int h = bh % p.H, b = bh / p.H;
  uint8_t* row = p.maskx + (int64_t)rowid * 2 * p.N;
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
  for (int n = threadIdx.x; n < p.N; n += blockDim.x) row[p.N + n] = row[n] ^ 1;
  if (rowid == 0)
    for (int n = threadIdx.x; n < p.N; n += blockDim.x)
      p.kvvx[n] = p.kvvx[p.N + n] = min(p.bk, p.Sk - n * p.bk);
}

// Gradients out of the extended problem: dk, dv for rows t < Sk; the mean
// key's gradient c_n * dK of block n's first copy and the summed value's
// dV of that copy.  Rows B*Sk*Hkv of dk/dv first, then B*N*Hkv summary rows.
__global__ __launch_bounds__(256) void proxy_gather_kernel(ProxyBwdParams p, int64_t chunks) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= chunks) return;
  const int cpr = p.D / 8;
  const int64_t row = c / cpr;
  const int d0 = (int)(c % cpr) * 8;
  const int64_t Sx = 2 * (int64_t)p.N * p.bk;
  const int64_t tok_rows = (int64_t)p.B * p.Sk * p.Hkv;
  if (row < tok_rows) {
    const int hk = (int)(row % p.Hkv);
    const int64_t bt = row / p.Hkv;
    const int t = (int)(bt % p.Sk), b = (int)(bt / p.Sk);
    const int64_t src = (((int64_t)b * Sx + t) * p.Hkv + hk) * p.D + d0;
    *reinterpret_cast<uint4*>(p.dk + b * p.k_sb + (int64_t)t * p.k_ss + hk * p.k_sh + d0) =
        *reinterpret_cast<const uint4*>(p.dkx + src);
    *reinterpret_cast<uint4*>(p.dv + b * p.v_sb + (int64_t)t * p.v_ss + hk * p.v_sh + d0) =
        *reinterpret_cast<const uint4*>(p.dvx + src);
  } else {
    const int64_t r = row - tok_rows;
    const int hk = (int)(r % p.Hkv);
    const int64_t bn = r / p.Hkv;
    const int n = (int)(bn % p.N), b = (int)(bn / p.N);
    const float cn = (float)min(p.bk, p.Sk - n * p.bk);
    const int64_t t = (int64_t)p.N * p.bk + (int64_t)n * p.bk;  // the first copy
    const int64_t src = (((int64_t)b * Sx + t) * p.Hkv + hk) * p.D + d0;
    const uint4 g = *reinterpret_cast<const uint4*>(p.dkx + src);
    *reinterpret_cast<uint4*>(p.dks + b * p.ks_sb + (int64_t)n * p.ks_sn + hk * p.ks_sh + d0) =
        make_uint4(pack_bf16x2(bf_lo(g.x) * cn, bf_hi(g.x) * cn),
                   pack_bf16x2(bf_lo(g.y) * cn, bf_hi(g.y) * cn),
                   pack_bf16x2(bf_lo(g.z) * cn, bf_hi(g.z) * cn),
                   pack_bf16x2(bf_lo(g.w) * cn, bf_hi(g.w) * cn));
    *reinterpret_cast<uint4*>(p.dvs + b * p.vs_sb + (int64_t)n * p.vs_sn + hk * p.vs_sh + d0) =
        *reinterpret_cast<const uint4*>(p.dvx + src);
  }
}

}  // namespace

hipError_t launch_proxy_bwd_prepare(const ProxyBwdParams& p, hipStream_t s) {
  const int64_t chunks = (int64_t)p.B * 2 * p.N * p.bk * p.Hkv * (p.D / 8);
  if (chunks > 0)
    hipLaunchKernelGGL(proxy_expand_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0,
                       s, p, chunks);
  const int64_t rows = (int64_t)p.B * p.H * p.M;
  if (rows > 0)
    hipLaunchKernelGGL(proxy_ext_mask_kernel, dim3((unsigned)rows), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_proxy_bwd_gather(const ProxyBwdParams& p, hipStream_t s) {
  const int64_t chunks = ((int64_t)p.B * p.Sk * p.Hkv + (int64_t)p.B * p.N * p.Hkv) * (p.D / 8);
  if (chunks > 0)
    hipLaunchKernelGGL(proxy_gather_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0,
                       s, p, chunks);
  return hipGetLastError();
}

}  // namespace bsa
