// attn_qk_prep: the producer of Q and K, with the attention's norms in its
// epilogue.
//
// The bound softmax reads a small set of norms computed ahead of attention
// (vatt-ghern.pages.dev "deep-heygen-avatar-iv-trillium-tpu", section
// 拿掉 softmax 的序列相依), and the pages fuse producer stages so that each
// stage writes what the next reads, in the layout it reads it (cloudcurated
// "How is HeyGen optimizing AI video on Google Cloud TPUs", layout contracts
// after Wall 3).  This kernel is the last step that writes Q and K before
// attention in a video diffusion transformer:
//
//   per row x of one head (D values):  y = x * g / sqrt(mean(x^2) + eps)
//   rotary embedding of adjacent pairs: (y_2i, y_2i+1) turned by the angle
//       whose cos / sin the per-token tables give
//   bf16 out (nearest even), written through the output strides
//
// and, from the rounded rows it has just written, the outputs of attn_norms:
// |q_n|, the max |k_n| of each 16-key granule and (by the same small
// reduction kernel attn_norms uses) the per-head maxima.  That spares the
// attention step its separate read of Q and K.
//
// HBM-bound.  A row of D bf16 is handled by D/8 consecutive lanes, 16 bytes
// (8 elements, 4 rotary pairs) each, so the rotation needs no lane exchange
// and one wave-wide access moves 1 KiB.  A wave keeps the rotary table rows
// of its granule in registers and walks the heads, so the tables (shared by
// every head) are read from HBM once.  Arithmetic is fp32 with one rounding
// to bf16.
#include "bsvf_device.h"
#include "bsvf_internal.h"

namespace bsvf {
namespace {

constexpr int kPrepThreads = 256;
constexpr int kPrepWaves = kPrepThreads / 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct PrepArgs {
  const u16* qi;
  const u16* ki;
  u16* qo;
  u16* ko;
  int64_t s[4][3];  // element strides {b, h, n} of qi, ki, qo, ko
  const float* gq;
  const float* gk;
  const float* cos;
  const float* sin;
  float eps;
  int32_t H, N;
  float* q_norm;
  float* k_gmax;
  float* head_max;
};

// One row chunk through the producer: 8 elements x (bf16 bits in w), weights
// g, rotary cos/sin of the chunk's 4 pairs.  Returns the packed bf16 result
// and, in ss_out, this lane's share of the rounded row's sum of squares.
template <int LPR>
__device__ __forceinline__ u32x4 prep_chunk(u32x4 w, const float (&g)[8], f32x4 c, f32x4 s, float eps,
                                            float inv_d, float& ss_out) {
  float x[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf16lo(w[e]);
    x[2 * e + 1] = bf16hi(w[e]);
  }
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
  const float r = 1.0f / __builtin_sqrtf(fmaf(ss, inv_d, eps));
  u32x4 out;
  float so = 0.0f;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float a = x[2 * p] * r * g[2 * p], b = x[2 * p + 1] * r * g[2 * p + 1];
    f32x2 z = {a * c[p] - b * s[p], a * s[p] + b * c[p]};
    const uint32_t bits = __builtin_bit_cast(uint32_t, __builtin_convertvector(z, bf16x2));
    out[p] = bits;
    const float z0 = bf16lo(bits), z1 = bf16hi(bits);
    so = fmaf(z0, z0, so);
    so = fmaf(z1, z1, so);
  }
  ss_out = so;
  return out;
}

// A workgroup covers kPrepWaves consecutive 16-row granules of one batch
// entry, one per wave, for every head.  A wave loads the rotary table rows of
// its granule once, keeps them in registers and walks the heads.
template <int D, bool NORMS>
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(PrepArgs a) {
  constexpr int LPR = D / 8;     // lanes per row
  constexpr int RPI = 64 / LPR;  // rows per wave-wide access
  constexpr int IPG = 16 / RPI;  // accesses per 16-row granule
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.y;
  const int G = a.N / 16;
  const int g = blockIdx.x * kPrepWaves + wave;
  const int c = lane % LPR, rsub = lane / LPR;
  const float inv_d = 1.0f / D;

  // the head-max pass that follows merges into a cleared head_max
  if (NORMS && blockIdx.x == 0)
    for (int h = threadIdx.x; h < 2 * a.H; h += kPrepThreads) a.head_max[2 * b * a.H + h] = 0.0f;
  if (g >= G) return;
  float gq[8], gk[8];
  {
    const f32x4 q0 = *reinterpret_cast<const f32x4*>(a.gq + 8 * c);
    const f32x4 q1 = *reinterpret_cast<const f32x4*>(a.gq + 8 * c + 4);
    const f32x4 k0 = *reinterpret_cast<const f32x4*>(a.gk + 8 * c);
    const f32x4 k1 = *reinterpret_cast<const f32x4*>(a.gk + 8 * c + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { gq[e] = q0[e]; gq[4 + e] = q1[e]; gk[e] = k0[e]; gk[4 + e] = k1[e]; }
  }
  f32x4 cv[IPG], sv[IPG];
#pragma unroll
  for (int it = 0; it < IPG; ++it) {
    const int row = g * 16 + it * RPI + rsub;
    cv[it] = *reinterpret_cast<const f32x4*>(a.cos + (int64_t)row * (D / 2) + 4 * c);
    sv[it] = *reinterpret_cast<const f32x4*>(a.sin + (int64_t)row * (D / 2) + 4 * c);
  }
  auto load = [&](int h, u32x4 (&qv)[IPG], u32x4 (&kv)[IPG]) {
    const u16* qi = a.qi + b * a.s[0][0] + h * a.s[0][1];
    const u16* ki = a.ki + b * a.s[1][0] + h * a.s[1][1];
#pragma unroll
    for (int it = 0; it < IPG; ++it) {
      const int row = g * 16 + it * RPI + rsub;
      qv[it] = *reinterpret_cast<const u32x4*>(qi + (int64_t)row * a.s[0][2] + 8 * c);
      kv[it] = *reinterpret_cast<const u32x4*>(ki + (int64_t)row * a.s[1][2] + 8 * c);
    }
  };
  auto work = [&](int h, const u32x4 (&qv)[IPG], const u32x4 (&kv)[IPG]) {
    u16* qo = a.qo + b * a.s[2][0] + h * a.s[2][1];
    u16* ko = a.ko + b * a.s[3][0] + h * a.s[3][1];
    const int64_t bh = (int64_t)b * a.H + h;
    float kg = 0.0f;
#pragma unroll
    for (int it = 0; it < IPG; ++it) {
      const int row = g * 16 + it * RPI + rsub;
      float sq, sk;
      const u32x4 qr = prep_chunk<LPR>(qv[it], gq, cv[it], sv[it], a.eps, inv_d, sq);
      const u32x4 kr = prep_chunk<LPR>(kv[it], gk, cv[it], sv[it], a.eps, inv_d, sk);
      *reinterpret_cast<u32x4*>(qo + (int64_t)row * a.s[2][2] + 8 * c) = qr;
      *reinterpret_cast<u32x4*>(ko + (int64_t)row * a.s[3][2] + 8 * c) = kr;
      if constexpr (NORMS) {
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) {
          sq += __shfl_xor(sq, m);
          sk += __shfl_xor(sk, m);
        }
        const float qn = __builtin_sqrtf(sq), kn = __builtin_sqrtf(sk);
        if (c == 0) a.q_norm[bh * a.N + row] = qn;
        kg = fmaxf(kg, kn);
      }
    }
    if constexpr (NORMS) {
#pragma unroll
      for (int m = LPR; m < 64; m <<= 1) kg = fmaxf(kg, __shfl_xor(kg, m));
      if (lane == 0) a.k_gmax[bh * G + g] = kg;
    }
  };
#pragma unroll 1
  for (int h = 0; h < a.H; ++h) {
    u32x4 qv[IPG], kv[IPG];
    load(h, qv, kv);
    work(h, qv, kv);
  }
}

template <int D, bool NORMS>
void prep_launch(const PrepArgs& a, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((prep_kernel<D, NORMS>), grid, dim3(kPrepThreads), 0, stream, a);
}

bool same_strides(const int64_t* x, const int64_t* y) { return x[0] == y[0] && x[1] == y[1] && x[2] == y[2]; }

}  // namespace
}  // namespace bsvf

using namespace bsvf;

extern "C" int attn_qk_prep(const void* q_in, const void* k_in, void* q_out, void* k_out, int32_t batch,
                            int32_t heads, int32_t seq_len, int32_t head_dim, const int64_t* strides,
                            const float* q_gamma, const float* k_gamma, float eps, const float* rope_cos,
                            const float* rope_sin, float* q_norm, float* k_gmax, float* head_max,
                            hipStream_t stream) {
  if (batch <= 0 || heads <= 0 || seq_len <= 0) return fail(ATTN_E_INVAL, "sizes must be positive");
  if (head_dim != 64 && head_dim != 128) return fail(ATTN_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (seq_len % 16) return fail(ATTN_E_ALIGN, "seq_len must be a multiple of 16");
  if (!strides) return fail(ATTN_E_INVAL, "strides must not be NULL");
  int st;
  if ((st = check_tensor("q_in", q_in, strides, batch, heads, seq_len, head_dim))) return st;
  if ((st = check_tensor("k_in", k_in, strides + 3, batch, heads, seq_len, head_dim))) return st;
  if ((st = check_tensor("q_out", q_out, strides + 6, batch, heads, seq_len, head_dim))) return st;
  if ((st = check_tensor("k_out", k_out, strides + 9, batch, heads, seq_len, head_dim))) return st;
  if ((q_out == q_in && !same_strides(strides + 6, strides)) || (k_out == k_in && !same_strides(strides + 9, strides + 3)))
    return fail(ATTN_E_INVAL, "an output may replace its input only with identical strides");
  if (q_out == k_out || q_out == k_in || k_out == q_in)
    return fail(ATTN_E_INVAL, "q_out and k_out must not alias each other or the other input");
  if (!q_gamma || !k_gamma || !rope_cos || !rope_sin)
    return fail(ATTN_E_INVAL, "weights and rotary tables must not be NULL");
  if (!aligned16(q_gamma) || !aligned16(k_gamma) || !aligned16(rope_cos) || !aligned16(rope_sin))
    return fail(ATTN_E_ALIGN, "weights and rotary tables must be 16-byte aligned");
  if (!(eps >= 0.0f) || !(eps <= 3.0e38f)) return fail(ATTN_E_INVAL, "eps must be finite and >= 0");
  const int n_norm = (q_norm != nullptr) + (k_gmax != nullptr) + (head_max != nullptr);
  if (n_norm != 0 && n_norm != 3) return fail(ATTN_E_INVAL, "norm outputs must be all given or all NULL");
  if ((int64_t)batch * heads > 65535) return fail(ATTN_E_SIZE, "batch * heads exceeds 65535");
  if ((int64_t)batch * heads * seq_len > (int64_t)1 << 40) return fail(ATTN_E_SIZE, "too many rows");

  PrepArgs a;
  a.qi = static_cast<const u16*>(q_in);
  a.ki = static_cast<const u16*>(k_in);
  a.qo = static_cast<u16*>(q_out);
  a.ko = static_cast<u16*>(k_out);
  for (int t = 0; t < 4; ++t)
    for (int j = 0; j < 3; ++j) a.s[t][j] = strides[3 * t + j];
  a.gq = q_gamma;
  a.gk = k_gamma;
  a.cos = rope_cos;
  a.sin = rope_sin;
  a.eps = eps;
  a.H = heads;
  a.N = seq_len;
  const int granules = seq_len / 16;
  const int blocks = (granules + kPrepWaves - 1) / kPrepWaves;
  a.q_norm = q_norm;
  a.k_gmax = k_gmax;
  a.head_max = head_max;
  const dim3 grid(blocks, batch);
  const bool norms = n_norm == 3;
  if (head_dim == 128) {
    if (norms) prep_launch<128, true>(a, grid, stream);
    else prep_launch<128, false>(a, grid, stream);
  } else {
    if (norms) prep_launch<64, true>(a, grid, stream);
    else prep_launch<64, false>(a, grid, stream);
  }
  if (norms) launch_head_max(q_norm, k_gmax, batch * heads, seq_len, head_max, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ATTN_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
  return bsvf::ok();
}
