// band_prefill_attn: causal, keep-set-masked attention over whole sequences,
// bf16 in, fp32 accumulation, on the matrix cores (v_mfma_f32_16x16x32_bf16).
//
// Workgroup = 4 waves = BM = 64*RB query rows of one (batch, head); each wave
// owns 16*RB rows.  Key tiles of 64 rows are staged in LDS -- K row-major,
// V transposed -- while the next kept tile is already being fetched into
// registers.  Scores are computed transposed, S^T = K Q^T (A = K from LDS,
// B = Q^T from registers), so that the MFMA result gives every lane one query
// row and four keys of each 16-key block.  That lane-per-row layout is kept
// for the whole softmax: the running max/sum are per lane (combined over the
// four lanes of a row by two xor shuffles), the probabilities P^T are
// already in the B-operand layout of the second product, and the output is
// accumulated transposed, O^T += V^T P^T (A = V^T from LDS), so the online
// rescale is one multiply per lane register.  The contraction index of both
// products is assigned to lanes the same way on both operands, which is all
// the MFMA needs.
//
// Sparsity: a 64-key tile is visited only if some (row, key) pair in it is
// kept; inside a visited tile each wave skips 16-key blocks with no kept
// pair for its rows, and element masks are applied only to blocks that are
// not entirely kept.  Workgroups are numbered so that all query tiles of one
// (batch, head) share an XCD (hardware dispatches workgroups to the 8 XCDs
// round-robin), which keeps the prompt keys/values every tile re-reads in
// that XCD's L2.
#include "common.h"

namespace da {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;                       // [batch][heads][n] or null
  int64_t sq[3], sk[3], sv[3], so[3];   // element strides (batch, head, position)
  const int32_t* prompt_len;        // [batch]
  int batch, heads, kv_heads, n, n_qt;
  int mode, W, B, G;
  float qscale;                     // scale * log2(e)
};

constexpr int BN = 64;              // keys per tile
constexpr float kLog2eP = 1.4426950408889634f;
constexpr float kLn2P = 0.6931471805599453f;

// Does any pair (i, j), i in [ilo, ihi], j in [jlo, jhi], pass the causal
// keep rule?  (Exact; used to skip tiles and blocks.)
__device__ inline bool range_has_kept(int ilo, int ihi, int jlo, int jhi, int P, int mode, int W,
                                      int B, int G) {
  if (jlo > ihi) return false;                   // causal
  if (mode == DA_MODE_DENSE) return true;
  if (jlo < P) return true;                      // a prompt key under the diagonal
  const int dlo = ilo - jhi > 0 ? ilo - jhi : 0;
  const int dhi = ihi - jlo < W ? ihi - jlo : W;
  if (dlo > dhi) return false;
  if (mode == DA_MODE_BAND) return dlo <= B;
  if (2 * B + 1 >= G) return true;
  const int r = dlo % G;
  if (r <= B || r >= G - B) return true;
  return dlo - r + G - B <= dhi;                 // next band start
}

// Is every pair in the range kept (no element mask needed)?
__device__ inline bool range_all_kept(int ilo, int jhi, int P, int mode) {
  if (jhi > ilo) return false;                   // causal: every key <= every row
  return mode == DA_MODE_DENSE || jhi < P;
}

__device__ inline bool keep_pair(int i, int j, int P, int mode, int W, int B, int G) {
  if (j > i) return false;
  if (mode == DA_MODE_DENSE || j < P) return true;
  const int d = i - j;
  return d <= W && window_keep(mode, d, B, G);
}

template <int HD, int RB>
__global__ void __launch_bounds__(256) prefill_kernel(PrefillArgs a) {
  constexpr int BM = 64 * RB;
  constexpr int NC = HD / 32;        // 32-wide contraction chunks of the head dim
  constexpr int NB = HD / 16;        // 16-wide output blocks of the head dim
  constexpr int KSTR = HD + 8;       // LDS row stride of K (elements), padded
  constexpr int VSTR = BN + 4;       // LDS row stride of V^T (elements), padded
  constexpr int CPR = HD / 8;        // 16-byte chunks per key row
  constexpr int LPT = BN * CPR / 256;  // 16-byte chunks per thread per tile (K and V each)

  __shared__ __attribute__((aligned(16))) uint16_t ks[BN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t vt[HD * VSTR];

  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  const int lr = lane & 15;          // row (or column) within a 16-block
  const int lg = lane >> 4;          // lane group 0..3

  const int n_bh = a.batch * a.heads;
  const int bh = blockIdx.x % n_bh;  // all query tiles of (b, h) on one XCD
  const int qt = blockIdx.x / n_bh;
  const int b = bh / a.heads;
  const int h = bh % a.heads;
  const int hk = h / (a.heads / a.kv_heads);
  const int i0 = qt * BM;
  const int n = a.n;
  const int P = clampi(a.prompt_len[b], 0, n);
  const int i_last = i0 + BM - 1 < n - 1 ? i0 + BM - 1 : n - 1;

  const uint16_t* qb = a.q + b * a.sq[0] + h * a.sq[1];
  const uint16_t* kb = a.k + b * a.sk[0] + hk * a.sk[1];
  const uint16_t* vb = a.v + b * a.sv[0] + hk * a.sv[1];

  // ---- this wave's query rows: 16*RB, lane lr of block rb holds row
  // wi0 + 16*rb + lr; Q^T operand chunks kept in registers
  const int wi0 = i0 + wave * 16 * RB;
  bf16x8 qv[RB][NC];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int i = wi0 + 16 * rb + lr;
    const uint16_t* qrow = qb + (int64_t)(i < n ? i : n - 1) * a.sq[2];
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qv[rb][c] = *reinterpret_cast<const bf16x8*>(qrow + 32 * c + lg * 8);
  }

  float m[RB], ls[RB];
  f32x4 o[RB][NB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = -INFINITY;
    ls[rb] = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- kept key tiles of this query tile, in order
  const int jt_hi = i_last / BN;
  auto next_tile = [&](int jt) {
    for (++jt; jt <= jt_hi; ++jt)
      if (range_has_kept(i0, i_last, jt * BN, jt * BN + BN - 1, P, a.mode, a.W, a.B, a.G)) break;
    return jt;
  };

  // global -> registers for one tile: thread t moves LPT 16-byte chunks of K
  // and of V; rows past the sequence end re-read row n-1 (masked later)
  u32x4 pk[LPT], pv[LPT];
  auto fetch = [&](int jt) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int idx = u * 256 + t;
      const int kr = idx / CPR, ch = idx % CPR;
      int j = jt * BN + kr;
      j = j < n ? j : n - 1;
      pk[u] = *reinterpret_cast<const u32x4*>(kb + (int64_t)j * a.sk[2] + ch * 8);
      pv[u] = *reinterpret_cast<const u32x4*>(vb + (int64_t)j * a.sv[2] + ch * 8);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int idx = u * 256 + t;
      const int kr = idx / CPR, ch = idx % CPR;
      *reinterpret_cast<u32x4*>(ks + kr * KSTR + ch * 8) = pk[u];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = pv[u][e];
        vt[(ch * 8 + 2 * e) * VSTR + kr] = (uint16_t)(w & 0xffffu);
        vt[(ch * 8 + 2 * e + 1) * VSTR + kr] = (uint16_t)(w >> 16);
      }
    }
  };

  int jt = next_tile(-1);
  if (jt <= jt_hi) fetch(jt);
  while (jt <= jt_hi) {
    __syncthreads();                 // every wave is done with the previous tile
    stage();
    __syncthreads();
    const int jn = next_tile(jt);
    if (jn <= jt_hi) fetch(jn);      // in flight while this tile computes
    const int j0 = jt * BN;

#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rlo = wi0 + 16 * rb;
      const int rhi = rlo + 15 < i_last ? rlo + 15 : i_last;
      if (rlo > i_last) continue;
      const int i = rlo + lr;        // this lane's row
      // ---- S^T blocks (16 keys each), scaled to the log2 domain
      f32x4 s[4];
      bool need[4];
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4) {
        const int jlo = j0 + 16 * kb4;
        need[kb4] = range_has_kept(rlo, rhi, jlo, jlo + 15, P, a.mode, a.W, a.B, a.G);
        s[kb4] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (need[kb4]) {
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + (16 * kb4 + lr) * KSTR + 32 * c + lg * 8);
            s[kb4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qv[rb][c], s[kb4], 0, 0, 0);
          }
          const bool full = range_all_kept(rlo, jlo + 15, P, a.mode);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = jlo + 4 * lg + r;
            const bool kp = full || (i < n && keep_pair(i, j, P, a.mode, a.W, a.B, a.G));
            s[kb4][r] = kp ? s[kb4][r] * a.qscale : -INFINITY;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) s[kb4][r] = -INFINITY;
        }
      }
      // ---- online softmax for this lane's row
      float mt = -INFINITY;
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
        for (int r = 0; r < 4; ++r) mt = fmaxf(mt, s[kb4][r]);
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mn = fmaxf(m[rb], mt);
      const float mref = mn == -INFINITY ? 0.f : mn;
      const float alpha = exp2f(m[rb] - mref);
      m[rb] = mn;
      ls[rb] *= alpha;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[rb][nb][r] *= alpha;
      // P^T as the B operand of O^T += V^T P^T: slot e of 32-key chunk cc is
      // key 32cc + (e/4)*16 + 4*lg + e%4, i.e. block 2cc+e/4, element e%4
      bf16x8 pb[2];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        uint16_t tmp[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = exp2f(s[2 * cc + e / 4][e % 4] - mref);
          ls[rb] += p;
          tmp[e] = (uint16_t)f32_to_bf16(p);
        }
        __builtin_memcpy(&pb[cc], tmp, 16);
      }
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        if (!need[2 * cc] && !need[2 * cc + 1]) continue;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint16_t* vrow = vt + (16 * nb + lr) * VSTR + 32 * cc + 4 * lg;
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow);        // 8-byte aligned
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
          const u32x4 w = u32x4{lo.x, lo.y, hi.x, hi.y};
          const bf16x8 vf = __builtin_bit_cast(bf16x8, w);
          o[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[cc], o[rb][nb], 0, 0, 0);
        }
      }
    }
    jt = jn;
  }

  // ---- normalise and store: lane holds row rlo+lr, dims 16nb + 4lg + r
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float L = ls[rb];
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
    const int i = wi0 + 16 * rb + lr;
    if (i > i_last) continue;
    const float inv = 1.f / L;
    uint16_t* orow = a.o + b * a.so[0] + h * a.so[1] + (int64_t)i * a.so[2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint32_t w0 = f32_to_bf16(o[rb][nb][0] * inv) | (f32_to_bf16(o[rb][nb][1] * inv) << 16);
      const uint32_t w1 = f32_to_bf16(o[rb][nb][2] * inv) | (f32_to_bf16(o[rb][nb][3] * inv) << 16);
      *reinterpret_cast<uint2*>(orow + 16 * nb + 4 * lg) = make_uint2(w0, w1);
    }
    if (a.lse && lg == 0)
      a.lse[((int64_t)b * a.heads + h) * n + i] = (m[rb] + log2f(L)) * kLn2P;
  }
}

}  // namespace da

using namespace da;

extern "C" int da_band_prefill_attn(const da_mask* m, da_dtype dtype, int32_t batch, int32_t heads,
                                    int32_t kv_heads, int32_t n, int32_t head_dim,
                                    const void* q, const void* k, const void* v, void* out,
                                    const int64_t* strides, const int32_t* prompt_len,
                                    float scale, float* lse, void* stream) {
  int rc = check_mask(m);
  if (rc) return rc;
  if (!m->causal) return fail(DA_ENOTSUP, "prefill needs a causal mask");
  if (dtype != DA_BF16) return fail(DA_ENOTSUP, "prefill runs on bf16 inputs (dtype %d)", (int)dtype);
  if (head_dim != 64 && head_dim != 128) return fail(DA_ENOTSUP, "head_dim %d not in {64, 128}", head_dim);
  if (batch < 0 || heads < 1 || kv_heads < 1 || heads % kv_heads || n < 0)
    return fail(DA_EINVAL, "batch=%d heads=%d kv_heads=%d n=%d", batch, heads, kv_heads, n);
  if (!strides) return fail(DA_EINVAL, "strides is NULL");
  if (batch > 0 && n > 0 && (!q || !k || !v || !out || !prompt_len))
    return fail(DA_EINVAL, "q, k, v, out and prompt_len must be non-NULL");
  for (int i = 0; i < 12; ++i)
    if (strides[i] < 0 || (strides[i] * 2) % 16) return fail(DA_EINVAL, "stride %d must be a non-negative multiple of 8 elements", i);
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) % 16)
    return fail(DA_EINVAL, "q, k, v and out must be 16-byte aligned");
  clear_error();
  if (batch == 0 || n == 0) return DA_OK;
  PrefillArgs a;
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.k = reinterpret_cast<const uint16_t*>(k);
  a.v = reinterpret_cast<const uint16_t*>(v);
  a.o = reinterpret_cast<uint16_t*>(out);
  a.lse = lse;
  for (int i = 0; i < 3; ++i) {
    a.sq[i] = strides[i];
    a.sk[i] = strides[3 + i];
    a.sv[i] = strides[6 + i];
    a.so[i] = strides[9 + i];
  }
  a.prompt_len = prompt_len;
  a.batch = batch;
  a.heads = heads;
  a.kv_heads = kv_heads;
  a.n = n;
  a.mode = m->mode;
  a.W = m->W;
  a.B = m->B;
  a.G = m->G;
  a.qscale = scale * kLog2eP;
  constexpr int RB = 1;
  const int bm = 64 * RB;
  a.n_qt = (n + bm - 1) / bm;
  const int64_t blocks = (int64_t)a.n_qt * batch * heads;
  if (blocks > 0x7fffffff) return fail(DA_ENOTSUP, "grid too large");
  if (head_dim == 128)
    hipLaunchKernelGGL((prefill_kernel<128, RB>), dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<64, RB>), dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a);
  return check_launch("prefill_kernel");
}
