// moe_oracle.cpp -- plain, slow CPU oracle for the routed-expert MoE forward.
//
// TEST INFRASTRUCTURE ONLY. Nothing on the product path may load this file's
// library: only the tests, the smoke entry point and the benchmark's CPU
// baseline leg use it. It shares no code, header, table or helper with the HIP
// library; it includes only the C++ standard library and OpenMP.
//
// What it computes (sources, by page title and section):
//   [A] "tilelang baseline" MoE walkthrough (devpress.csdn.net, tilelang-metax
//       race): section "forward" (expert sort, counts, offsets, padded offsets,
//       block->expert table), section "stage-1 gate+up" (SiLU(gate)*up),
//       section "stage-2 down".
//   [B] TileLang tutorial ch.18 "End-to-end II", skeletons.py,
//       moe_routed_kernel docstring (the dispatch contract) and body.
//   [C] TileOPs-Metax PR #55 "moe_reduce_fused", section 1 (optimisation plan:
//       fp32 accumulation, K order kept, pos < 0 skipped) and section 2
//       (reference semantics, with_weights=False means all-ones weights).
//
// Precision: the pages fix fp32 accumulation ([A] stage-1/2 accum dtype,
// [C] section 1), so every dot product and the weighted sum accumulate in
// fp32 with fused multiply-add, in ascending index order. The intermediates
// h = SiLU(g)*u and expert_out are tensors of the activation dtype in [B]
// (UpLogits / Output), so for 16-bit dtypes they are rounded
// (round-to-nearest-even) to that dtype at exactly those two points. With the
// fp32 dtype no rounding happens. The output y is returned in fp32.
//
// Parity pins for every exported function live in the CPU test-suite: a
// dense fp64 brute force without any dispatch, closed forms, invariants and
// the worked table examples of [A]. See oracle/__init__.py for the loader.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

#include <omp.h>

namespace {

// Storage codes of this file (an interface agreement with the tests only).
constexpr int kF16 = 0;
constexpr int kBF16 = 1;
constexpr int kF32 = 2;
constexpr int kFP8 = 3;   // OCP FP8 E4M3 "fn"

// ---------------------------------------------------------------- dtypes ---

// bfloat16 is the top half of an IEEE binary32; widening is exact.
float bf16_bits_to_float(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// binary32 -> bfloat16, round to nearest, ties to even. NaN stays NaN (quiet).
uint16_t float_to_bf16_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) {
    return static_cast<uint16_t>((u >> 16) | 0x0040u);
  }
  uint32_t keep = u >> 16;
  uint32_t rest = u & 0xffffu;
  if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
  return static_cast<uint16_t>(keep);
}

// IEEE binary16 -> binary32 (exact), written from the format definition:
// 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
float f16_bits_to_float(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int expo = (h >> 10) & 0x1f;
  const int frac = h & 0x3ff;
  float v;
  if (expo == 0) {
    v = std::ldexp(static_cast<float>(frac), -24);          // subnormal / zero
  } else if (expo == 31) {
    v = frac ? std::numeric_limits<float>::quiet_NaN()
             : std::numeric_limits<float>::infinity();
  } else {
    v = std::ldexp(static_cast<float>(frac | 0x400), expo - 25);
  }
  return sign ? -v : v;
}

// binary32 -> binary16, round to nearest, ties to even; overflow -> inf.
uint16_t float_to_f16_bits(float f) {
  const uint16_t sign = std::signbit(f) ? 0x8000u : 0u;
  if (std::isnan(f)) return static_cast<uint16_t>(sign | 0x7e00u);
  if (std::isinf(f)) return static_cast<uint16_t>(sign | 0x7c00u);
  const double a = std::fabs(static_cast<double>(f));
  if (a == 0.0) return sign;
  if (a < std::ldexp(1.0, -14)) {
    // Subnormal range: value = q * 2^-24 with integer q in [0, 1024].
    double q = std::nearbyint(a * std::ldexp(1.0, 24));    // ties to even
    return static_cast<uint16_t>(sign | static_cast<uint16_t>(q));
  }
  int e2;
  std::frexp(a, &e2);               // a = m * 2^e2, m in [0.5, 1)
  int unb = e2 - 1;                 // a in [2^unb, 2^(unb+1))
  double q = std::nearbyint(a * std::ldexp(1.0, 10 - unb));  // [1024, 2048]
  if (q >= 2048.0) { q = 1024.0; unb += 1; }
  if (unb > 15) return static_cast<uint16_t>(sign | 0x7c00u);
  const int biased = unb + 15;
  return static_cast<uint16_t>(sign | (biased << 10) | (static_cast<int>(q) - 1024));
}

// OCP FP8 E4M3 ("fn") -> binary32 (exact), from the format definition:
// 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits; exponent 0 holds
// subnormals; S.1111.111 is NaN; there are no infinities.
float fp8e4m3_bits_to_float(uint8_t b) {
  const int sign = (b >> 7) & 1;
  const int expo = (b >> 3) & 0xf;
  const int frac = b & 7;
  float v;
  if (expo == 15 && frac == 7) {
    v = std::numeric_limits<float>::quiet_NaN();
  } else if (expo == 0) {
    v = std::ldexp(static_cast<float>(frac), -9);
  } else {
    v = std::ldexp(static_cast<float>(frac | 8), expo - 10);
  }
  return sign ? -v : v;
}

// binary32 -> FP8 E4M3 "fn", round to nearest even; magnitudes at or above
// the largest finite value (448), infinities included, saturate to +-448.
uint8_t float_to_fp8e4m3_bits(float f) {
  const uint8_t sign = std::signbit(f) ? 0x80 : 0x00;
  if (std::isnan(f)) return static_cast<uint8_t>(sign | 0x7f);
  const double a = std::fabs(static_cast<double>(f));
  if (a >= 448.0) return static_cast<uint8_t>(sign | 0x7e);
  if (a < std::ldexp(1.0, -6)) {
    const double q = std::nearbyint(a * std::ldexp(1.0, 9));   // [0, 8]
    return static_cast<uint8_t>(sign | static_cast<int>(q));
  }
  int e2;
  std::frexp(a, &e2);
  int unb = e2 - 1;                                              // [-6, 8]
  double q = std::nearbyint(a * std::ldexp(1.0, 3 - unb));      // [8, 16]
  if (q >= 16.0) { q = 8.0; unb += 1; }
  return static_cast<uint8_t>(sign | ((unb + 7) << 3) | (static_cast<int>(q) - 8));
}

float load_elem(int dt, const void* base, int64_t i) {
  if (dt == kF32) return static_cast<const float*>(base)[i];
  if (dt == kFP8) return fp8e4m3_bits_to_float(static_cast<const uint8_t*>(base)[i]);
  const uint16_t b = static_cast<const uint16_t*>(base)[i];
  return dt == kBF16 ? bf16_bits_to_float(b) : f16_bits_to_float(b);
}

// Rounding of an fp32 value to the storage dtype and back ("mirror" rounding
// of the intermediates; identity for fp32).
float round_to(int dt, float v) {
  if (dt == kBF16) return bf16_bits_to_float(float_to_bf16_bits(v));
  if (dt == kF16) return f16_bits_to_float(float_to_f16_bits(v));
  return v;
}

bool dtype_ok(int dt) { return dt == kF16 || dt == kBF16 || dt == kF32; }
bool reduce_dtype_ok(int dt) { return dtype_ok(dt) || dt == kFP8; }

// SiLU(g) = g * sigmoid(g) = g / (1 + e^-g). [A] stage-1 writes sigmoid with
// exp2(-g*log2 e); the value is the same function, written here with expf.
float silu(float g) { return g / (1.0f + std::exp(-g)); }

// Expert weights as stored: dtype wdt (the activation dtype, or FP8 E4M3
// with one fp32 scale per weight row, i.e. per output channel: sg / su [E*D]
// for gate / up, sd [E*H] for down; NULL scales mean unscaled weights).
struct ExpertWeights {
  int wdt;
  const void* wg;
  const void* wu;
  const void* wd;
  const float* sg;
  const float* su;
  const float* sd;
};

// One routed pair: token row x_t against expert e.
//   g_j  = s_g[e,j] * sum_h Wg[e,j,h] x[h]   u_j = s_u[e,j] * sum_h Wu[e,j,h] x[h]
//   h_j  = R(SiLU(g_j) * u_j)                    ([A] stage-1 epilogue)
//   eo_c = R(s_d[e,c] * sum_j Wd[e,c,j] h_j)     ([A] stage-2, unweighted)
// (the scale factors apply to FP8 weights: each dot product runs over the
// decoded FP8 values, then is multiplied by its row's scale once). With
// row_w non-NULL the down output is weighted before its rounding,
//   eo_c = R(w * (s_d[e,c] * sum_j Wd[e,c,j] h_j)),  w = *row_w
// ([B] moe_routed_kernel: the down kernel multiplies each output row by the
// row's routing weight before writing it). W_gate /
// W_up are [E, D, H] and W_down is [E, H, D], row-major, so each dot product
// walks a contiguous row ([A] "forward": stacked expert weights).
void expert_pair(int dt, const float* xrow, const ExpertWeights& W, int e, int H, int D,
                 float* hbuf, float* eo, const float* row_w = nullptr) {
  for (int j = 0; j < D; ++j) {
    const int64_t row = (static_cast<int64_t>(e) * D + j) * H;
    float g = 0.0f, u = 0.0f;
    for (int k = 0; k < H; ++k) {
      g = std::fma(load_elem(W.wdt, W.wg, row + k), xrow[k], g);
      u = std::fma(load_elem(W.wdt, W.wu, row + k), xrow[k], u);
    }
    if (W.sg) g = g * W.sg[static_cast<int64_t>(e) * D + j];
    if (W.su) u = u * W.su[static_cast<int64_t>(e) * D + j];
    hbuf[j] = round_to(dt, silu(g) * u);
  }
  for (int c = 0; c < H; ++c) {
    const int64_t row = (static_cast<int64_t>(e) * H + c) * D;
    float o = 0.0f;
    for (int j = 0; j < D; ++j) o = std::fma(load_elem(W.wdt, W.wd, row + j), hbuf[j], o);
    if (W.sd) o = o * W.sd[static_cast<int64_t>(e) * H + c];
    if (row_w) o = o * *row_w;
    eo[c] = round_to(dt, o);
  }
}

// The full forward over a token list (see oracle_moe_forward). With
// weighted_down the routing weight is applied in the down output (above) and
// the combine is a plain fp32 sum in k order; otherwise the combine is the
// fma of each weight with the unweighted output, in k order.
int moe_forward(int dt, const void* x, const ExpertWeights& W, const int32_t* ids,
                const float* w, int T, int H, int D, int E, int K, const int32_t* tokens,
                int n_tokens, float* y, float* h_pairs, float* eo_pairs,
                bool weighted_down = false) {
  if (!dtype_ok(dt) || T < 0 || H <= 0 || D <= 0 || E <= 0 || K <= 0) return -1;
  if (!tokens && n_tokens != T) return -1;
  for (int i = 0; i < n_tokens; ++i) {
    const int t = tokens ? tokens[i] : i;
    if (t < 0 || t >= T) return -1;
    for (int k = 0; k < K; ++k) {
      if (ids[static_cast<int64_t>(t) * K + k] >= E) return -1;
    }
  }
#pragma omp parallel
  {
    std::vector<float> xrow(H), hbuf(D), eo(H), acc(H);
#pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < n_tokens; ++i) {
      const int t = tokens ? tokens[i] : i;
      for (int c = 0; c < H; ++c) xrow[c] = load_elem(dt, x, static_cast<int64_t>(t) * H + c);
      for (int c = 0; c < H; ++c) acc[c] = 0.0f;
      for (int k = 0; k < K; ++k) {
        const int64_t slot = static_cast<int64_t>(t) * K + k;
        const int64_t out_slot = static_cast<int64_t>(i) * K + k;
        const int e = ids[slot];
        if (e < 0) {
          if (h_pairs) for (int j = 0; j < D; ++j) h_pairs[out_slot * D + j] = 0.0f;
          if (eo_pairs) for (int c = 0; c < H; ++c) eo_pairs[out_slot * H + c] = 0.0f;
          continue;
        }
        const float wk = w[slot];
        expert_pair(dt, xrow.data(), W, e, H, D, hbuf.data(), eo.data(),
                    weighted_down ? &wk : nullptr);
        if (weighted_down) {
          for (int c = 0; c < H; ++c) acc[c] = acc[c] + eo[c];
        } else {
          for (int c = 0; c < H; ++c) acc[c] = std::fma(wk, eo[c], acc[c]);
        }
        if (h_pairs) for (int j = 0; j < D; ++j) h_pairs[out_slot * D + j] = hbuf[j];
        if (eo_pairs) for (int c = 0; c < H; ++c) eo_pairs[out_slot * H + c] = eo[c];
      }
      for (int c = 0; c < H; ++c) y[static_cast<int64_t>(i) * H + c] = acc[c];
    }
  }
  return 0;
}

}  // namespace

extern "C" {

// Threads the OpenMP loops below use (reported with the CPU baseline).
int oracle_num_threads(void) { return omp_get_max_threads(); }

// Sets the OpenMP thread count of later calls (the CPU baseline's 1-thread
// timings); changes no arithmetic: every loop over tokens computes each
// token's values in the same order at any thread count.
int oracle_set_num_threads(int n) {
  if (n < 1) return -1;
  omp_set_num_threads(n);
  return 0;
}

// ------------------------------------------------------------ conversions --
// Element-wise storage conversions, exported so the tests can pin them
// against library conversions and hand-made tie cases.
int oracle_to_f32(int dt, const void* in, float* out, int64_t n) {
  if (!reduce_dtype_ok(dt)) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = load_elem(dt, in, i);
  return 0;
}

int oracle_from_f32(int dt, const float* in, void* out, int64_t n) {
  if (!reduce_dtype_ok(dt)) return -1;
  for (int64_t i = 0; i < n; ++i) {
    if (dt == kF32) static_cast<float*>(out)[i] = in[i];
    else if (dt == kFP8) static_cast<uint8_t*>(out)[i] = float_to_fp8e4m3_bits(in[i]);
    else if (dt == kBF16) static_cast<uint16_t*>(out)[i] = float_to_bf16_bits(in[i]);
    else static_cast<uint16_t*>(out)[i] = float_to_f16_bits(in[i]);
  }
  return 0;
}

int oracle_silu_mul(const float* g, const float* u, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = silu(g[i]) * u[i];
  return 0;
}

// ------------------------------------------------------------- dispatch ----
// Number of row blocks: ceil(P / BM) + E with P = T*K, counted over every
// slot even when some are masked ([A] "forward", kernel grid size M).
int64_t oracle_num_blocks(int T, int K, int E, int BM) {
  const int64_t P = static_cast<int64_t>(T) * K;
  return (P + BM - 1) / BM + E;
}

// Expert-sorted dispatch ([A] "forward" steps 2-5; [B] dispatch contract).
//   * pairs p = t*K + k are grouped by expert, stable in p (the page's
//     argsort leaves ties unspecified; a stable counting sort is the reading
//     taken here);
//   * a slot whose id is negative is masked: it is not counted, and its
//     position is -1 (it is then skipped by the reduce, [C] section 1);
//   * group_offsets = exclusive prefix sum of group_sizes;
//   * group_padded_offsets[0] = 0 and
//     group_padded_offsets[e] = group_padded_offsets[e-1]
//                               + ceil((group_sizes[e-1] + 1) / BM) * BM;
//   * block_expert[bx] = the last expert e with group_padded_offsets[e] <= bx*BM.
// Returns the number of valid pairs, or -1 when an id is >= E or an argument
// is out of range. Entries of the sorted arrays past the valid count are set
// to -1 (pair, token) and 0 (weight).
int64_t oracle_dispatch(const int32_t* ids, const float* w, int T, int K, int E,
                        int BM, int32_t* group_sizes, int32_t* group_offsets,
                        int32_t* group_padded_offsets, int32_t* block_expert,
                        int32_t* sorted_pair, int32_t* sorted_token,
                        float* sorted_weight, int32_t* pos) {
  if (T < 0 || K <= 0 || E <= 0 || BM <= 0) return -1;
  const int64_t P = static_cast<int64_t>(T) * K;
  for (int64_t p = 0; p < P; ++p) {
    if (ids[p] >= E) return -1;
  }
  std::vector<int64_t> cnt(E, 0);
  for (int64_t p = 0; p < P; ++p) {
    if (ids[p] >= 0) cnt[ids[p]] += 1;
  }
  std::vector<int64_t> off(E, 0);
  for (int e = 1; e < E; ++e) off[e] = off[e - 1] + cnt[e - 1];
  int64_t n_valid = 0;
  for (int e = 0; e < E; ++e) n_valid += cnt[e];

  std::vector<int64_t> fill(E, 0);
  for (int64_t p = 0; p < P; ++p) {
    const int e = ids[p];
    if (e < 0) {
      pos[p] = -1;
      continue;
    }
    const int64_t i = off[e] + fill[e]++;
    sorted_pair[i] = static_cast<int32_t>(p);
    sorted_token[i] = static_cast<int32_t>(p / K);
    sorted_weight[i] = w ? w[p] : 1.0f;
    pos[p] = static_cast<int32_t>(i);
  }
  for (int64_t i = n_valid; i < P; ++i) {
    sorted_pair[i] = -1;
    sorted_token[i] = -1;
    sorted_weight[i] = 0.0f;
  }

  std::vector<int64_t> padded(E, 0);
  for (int e = 1; e < E; ++e) {
    const int64_t need = cnt[e - 1] + 1;
    padded[e] = padded[e - 1] + ((need + BM - 1) / BM) * BM;
  }
  for (int e = 0; e < E; ++e) {
    group_sizes[e] = static_cast<int32_t>(cnt[e]);
    group_offsets[e] = static_cast<int32_t>(off[e]);
    group_padded_offsets[e] = static_cast<int32_t>(padded[e]);
  }
  const int64_t nblk = oracle_num_blocks(T, K, E, BM);
  for (int64_t bx = 0; bx < nblk; ++bx) {
    const int64_t start = bx * BM;
    int owner = 0;
    for (int e = 0; e < E; ++e) {
      if (padded[e] <= start) owner = e;
    }
    block_expert[bx] = owner;
  }
  return n_valid;
}

// ---------------------------------------------------- expert MLP per pair --
// h (length D) and expert_out (length H) of one (token, expert) pair, as fp32
// values after the dtype rounding described above.
int oracle_expert_pair(int dt, const void* x, const void* wg, const void* wu,
                       const void* wd, int token, int expert, int H, int D,
                       float* h_out, float* eo_out) {
  if (!dtype_ok(dt) || H <= 0 || D <= 0) return -1;
  std::vector<float> xrow(H);
  for (int k = 0; k < H; ++k) xrow[k] = load_elem(dt, x, static_cast<int64_t>(token) * H + k);
  const ExpertWeights W{dt, wg, wu, wd, nullptr, nullptr, nullptr};
  expert_pair(dt, xrow.data(), W, expert, H, D, h_out, eo_out);
  return 0;
}

// ---------------------------------------------------------- full forward ---
//   y[t, :] = sum over k ascending with ids[t,k] >= 0 of
//             w[t,k] * expert_out(t, ids[t,k])[:]
// accumulated in fp32 with fused multiply-add ([C] section 1: fp32
// accumulator, K order kept, masked slots skipped; the routing weight is
// applied once, here, as the reduce of [C] does).
// tokens: optional list of n_tokens token indices to evaluate (NULL = all T
// tokens, n_tokens must then equal T). y is [n_tokens, H] fp32. h_pairs
// ([n_tokens*K, D]) and eo_pairs ([n_tokens*K, H]) are optional per-slot
// intermediates in the same (token, k) order; masked slots get zeros.
// Parallel over tokens with OpenMP; each token's arithmetic is sequential,
// so the result does not depend on the thread count.
int oracle_moe_forward(int dt, const void* x, const void* wg, const void* wu,
                       const void* wd, const int32_t* ids, const float* w, int T,
                       int H, int D, int E, int K, const int32_t* tokens,
                       int n_tokens, float* y, float* h_pairs, float* eo_pairs) {
  const ExpertWeights W{dt, wg, wu, wd, nullptr, nullptr, nullptr};
  return moe_forward(dt, x, W, ids, w, T, H, D, E, K, tokens, n_tokens, y, h_pairs, eo_pairs);
}

// The forward with the routing weight applied in the down output and an
// unweighted combine ([B] moe_routed_kernel's down epilogue):
//   eo_p = R(w_p * (h_p . Wd[e]))   y[t] = sum over unmasked k ascending of eo_(t,k)
// (fp32 adds in k order). Same arguments and outputs as oracle_moe_forward;
// eo_pairs holds the weighted rows.
int oracle_moe_forward_weighted_down(int dt, const void* x, const void* wg, const void* wu,
                                     const void* wd, const int32_t* ids, const float* w, int T,
                                     int H, int D, int E, int K, const int32_t* tokens,
                                     int n_tokens, float* y, float* h_pairs, float* eo_pairs) {
  const ExpertWeights W{dt, wg, wu, wd, nullptr, nullptr, nullptr};
  return moe_forward(dt, x, W, ids, w, T, H, D, E, K, tokens, n_tokens, y, h_pairs, eo_pairs,
                     true);
}

// ------------------------------------------------ FP8 expert weights ------
// Quantised expert weights (the pages leave the scheme open; taken here: OCP
// FP8 E4M3 codes with one fp32 scale per weight row, i.e. per output
// channel, activations in their own dtype). Per row r of `rows` rows of
// `cols` values of dtype dt:
//   amax = max_k |w[r, k]|,  s[r] = amax / 448 (1 for an all-zero row),
//   q[r, k] = FP8(w[r, k] / s[r])   (fp32 division, round to nearest even,
//                                     saturating at +-448).
int oracle_quantize_fp8_rows(int dt, const void* w, int64_t rows, int cols, uint8_t* q,
                             float* scales) {
  if (!dtype_ok(dt) || rows < 0 || cols <= 0) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    float amax = 0.0f;
    for (int k = 0; k < cols; ++k) amax = std::fmax(amax, std::fabs(load_elem(dt, w, r * cols + k)));
    const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    scales[r] = s;
    for (int k = 0; k < cols; ++k) q[r * cols + k] = float_to_fp8e4m3_bits(load_elem(dt, w, r * cols + k) / s);
  }
  return 0;
}

// The forward with FP8 expert weights and per-row scales (x, h, expert_out
// and y as in oracle_moe_forward; see expert_pair for the scale placement).
int oracle_moe_forward_w8(int dt, const void* x, const uint8_t* wg8, const uint8_t* wu8,
                          const uint8_t* wd8, const float* sg, const float* su, const float* sd,
                          const int32_t* ids, const float* w, int T, int H, int D, int E, int K,
                          const int32_t* tokens, int n_tokens, float* y, float* h_pairs,
                          float* eo_pairs) {
  if (!sg || !su || !sd) return -1;
  const ExpertWeights W{kFP8, wg8, wu8, wd8, sg, su, sd};
  return moe_forward(dt, x, W, ids, w, T, H, D, E, K, tokens, n_tokens, y, h_pairs, eo_pairs);
}

}  // extern "C"

namespace {

// ------------------------------------------------------------- W4A8 -------
// Int4 weights with int8 activations ([B] w4a8_dequant_gemm: weights int4
// packed two per uint8, activations int8, int32 accumulation; [B] module
// docstring: the weight + activation mode, each side dequantised in the
// kernel). Storage of a packed row: element 2i in bits 0..3 of byte i,
// element 2i+1 in bits 4..7 ([B] the uint8 -> int4 unpack: the field at
// position j % 2 is shifted right by 4 * (j % 2)); a field is a 4-bit two's
// complement number in [-8, 7].
int int4_at(const uint8_t* row, int64_t k) {
  const int nib = (row[k >> 1] >> (4 * (k & 1))) & 0xF;
  return nib >= 8 ? nib - 16 : nib;
}

// Symmetric per-row quantisation (the scheme is left open by the pages;
// taken here): s = amax / qmax (1 for an all-zero row), q = the integer
// nearest to v / s (fp32 division, ties to even), clamped to [qmin, qmax].
template <typename Store>
void quantize_rows(int dt, const void* v, int64_t rows, int cols, float qmax, float qmin,
                   float* scales, Store store) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    float amax = 0.0f;
    for (int k = 0; k < cols; ++k) amax = std::fmax(amax, std::fabs(load_elem(dt, v, r * cols + k)));
    const float s = amax > 0.0f ? amax / qmax : 1.0f;
    scales[r] = s;
    for (int k = 0; k < cols; ++k) {
      float q = std::nearbyint(load_elem(dt, v, r * cols + k) / s);
      q = std::fmin(std::fmax(q, qmin), qmax);
      store(r, k, static_cast<int>(q));
    }
  }
}

}  // namespace

extern "C" {

// int8 activations: qmax = 127, codes in [-127, 127].
int oracle_quantize_int8_rows(int dt, const void* a, int64_t rows, int cols, int8_t* q,
                              float* scales) {
  if (!dtype_ok(dt) || rows < 0 || cols <= 0) return -1;
  quantize_rows(dt, a, rows, cols, 127.0f, -127.0f, scales,
                [&](int64_t r, int k, int v) { q[r * cols + k] = static_cast<int8_t>(v); });
  return 0;
}

// int4 weights: qmax = 7, codes in [-8, 7], packed as above ([rows, cols/2]).
int oracle_quantize_int4_rows(int dt, const void* w, int64_t rows, int cols, uint8_t* packed,
                              float* scales) {
  if (!dtype_ok(dt) || rows < 0 || cols <= 0 || cols % 2) return -1;
  const int64_t half = cols / 2;
  for (int64_t i = 0; i < rows * half; ++i) packed[i] = 0;
  quantize_rows(dt, w, rows, cols, 7.0f, -8.0f, scales, [&](int64_t r, int k, int v) {
    uint8_t& b = packed[r * half + k / 2];
    b = static_cast<uint8_t>(b | ((v & 0xF) << (4 * (k % 2))));
  });
  return 0;
}

// [B] w4a8_dequant_gemm: Ct[n, m] = sum_k A[m, k] * B4[n, k] with A int8
// [M, K], B packed int4 [N, K/2] and the int32 result written transposed,
// [N, M]. Summed exactly (int64 here); returns -2 if a result leaves the
// int32 range, which int32 accumulation could not represent.
int oracle_w4a8_gemm(const int8_t* A, const uint8_t* B, int M, int N, int K, int32_t* Ct) {
  if (M < 0 || N < 0 || K <= 0 || K % 2) return -1;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int n = 0; n < N; ++n) {
    const uint8_t* brow = B + static_cast<int64_t>(n) * (K / 2);
    for (int m = 0; m < M; ++m) {
      int64_t acc = 0;
      for (int k = 0; k < K; ++k) acc += static_cast<int64_t>(A[static_cast<int64_t>(m) * K + k]) * int4_at(brow, k);
      if (acc > INT32_MAX || acc < INT32_MIN) bad = 1;
      Ct[static_cast<int64_t>(n) * M + m] = static_cast<int32_t>(acc);
    }
  }
  return bad ? -2 : 0;
}

}  // extern "C"

namespace {

// Dequantised dot product: (float) acc * s_a * s_w, left to right in fp32.
float dequant(int64_t acc, float sa, float sw) { return static_cast<float>(acc) * sa * sw; }

}  // namespace

extern "C" {

// The forward with W4A8 experts: x [T, H] (dtype dt) quantised per token to
// int8 (oracle_quantize_int8_rows); per routed pair (token t, expert e):
//   g_j  = dequant(sum_h xq[t,h] Wg4[e,j,h], sx[t], sg[e,j]),  u_j likewise
//   h_j  = R(SiLU(g_j) * u_j)                     (dtype dt, as the 16-bit path)
//   hq   = int8 quantisation of the pair's h row, scale sh
//   eo_c = R(dequant(sum_j hq[j] Wd4[e,c,j], sh, sd[e,c]))
// then y[t] = the fp32 fma sum over k ascending of w[t,k] * eo (masked slots
// skipped), as oracle_moe_forward. Weights: packed int4 [E, D, H/2] (gate,
// up) and [E, H, D/2] (down) with fp32 row scales [E*D] / [E*H].
int oracle_moe_forward_w4a8(int dt, const void* x, const uint8_t* wg4, const uint8_t* wu4,
                            const uint8_t* wd4, const float* sg, const float* su, const float* sd,
                            const int32_t* ids, const float* w, int T, int H, int D, int E, int K,
                            const int32_t* tokens, int n_tokens, float* y, float* h_pairs,
                            float* eo_pairs) {
  if (!dtype_ok(dt) || T < 0 || H <= 0 || D <= 0 || E <= 0 || K <= 0 || H % 2 || D % 2) return -1;
  if (!tokens && n_tokens != T) return -1;
  for (int i = 0; i < n_tokens; ++i) {
    const int t = tokens ? tokens[i] : i;
    if (t < 0 || t >= T) return -1;
    for (int k = 0; k < K; ++k) {
      if (ids[static_cast<int64_t>(t) * K + k] >= E) return -1;
    }
  }
#pragma omp parallel
  {
    std::vector<int8_t> xq(H), hq(D);
    std::vector<float> hbuf(D), eo(H), acc(H);
#pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < n_tokens; ++i) {
      const int t = tokens ? tokens[i] : i;
      float sx = 0.0f;
      quantize_rows(dt, static_cast<const char*>(x) + static_cast<int64_t>(t) * H * (dt == kF32 ? 4 : 2),
                    1, H, 127.0f, -127.0f, &sx, [&](int64_t, int k, int v) { xq[k] = static_cast<int8_t>(v); });
      for (int c = 0; c < H; ++c) acc[c] = 0.0f;
      for (int k = 0; k < K; ++k) {
        const int64_t slot = static_cast<int64_t>(t) * K + k;
        const int64_t out_slot = static_cast<int64_t>(i) * K + k;
        const int e = ids[slot];
        if (e < 0) {
          if (h_pairs) for (int j = 0; j < D; ++j) h_pairs[out_slot * D + j] = 0.0f;
          if (eo_pairs) for (int c = 0; c < H; ++c) eo_pairs[out_slot * H + c] = 0.0f;
          continue;
        }
        for (int j = 0; j < D; ++j) {
          const int64_t row = static_cast<int64_t>(e) * D + j;
          int64_t ag = 0, au = 0;
          for (int c = 0; c < H; ++c) {
            ag += static_cast<int64_t>(xq[c]) * int4_at(wg4 + row * (H / 2), c);
            au += static_cast<int64_t>(xq[c]) * int4_at(wu4 + row * (H / 2), c);
          }
          const float g = dequant(ag, sx, sg[row]);
          const float u = dequant(au, sx, su[row]);
          hbuf[j] = round_to(dt, silu(g) * u);
        }
        float sh = 0.0f;
        quantize_rows(kF32, hbuf.data(), 1, D, 127.0f, -127.0f, &sh,
                      [&](int64_t, int j, int v) { hq[j] = static_cast<int8_t>(v); });
        for (int c = 0; c < H; ++c) {
          const int64_t row = static_cast<int64_t>(e) * H + c;
          int64_t ad = 0;
          for (int j = 0; j < D; ++j) ad += static_cast<int64_t>(hq[j]) * int4_at(wd4 + row * (D / 2), j);
          eo[c] = round_to(dt, dequant(ad, sh, sd[row]));
        }
        const float wk = w[slot];
        for (int c = 0; c < H; ++c) acc[c] = std::fma(wk, eo[c], acc[c]);
        if (h_pairs) for (int j = 0; j < D; ++j) h_pairs[out_slot * D + j] = hbuf[j];
        if (eo_pairs) for (int c = 0; c < H; ++c) eo_pairs[out_slot * H + c] = eo[c];
      }
      for (int c = 0; c < H; ++c) y[static_cast<int64_t>(i) * H + c] = acc[c];
    }
  }
  return 0;
}

// ------------------------------------------------------------- W8A8 -------
// FP8 weights against FP8 activations (the tutorial's module docstring: the
// weight + activation mode quantises both GEMM operands; the scheme is left
// open by the pages and taken here as the FP8 weights above with the same
// per-row E4M3 quantisation applied to the activations):
//   xq, sx: the E4M3 codes and scale of x[t] (oracle_quantize_fp8_rows of the
//           row: sx = amax / 448, codes = E4M3(x / sx))
//   g_j  = dequant_f(sum_h dec(xq[h]) * dec(Wg8[e,j,h]), sx, sg[e,j]),  u_j likewise
//          (the sum an fp32 fma chain over h ascending; each product of two
//          E4M3 values is exact in fp32)
//   h_j  = R(SiLU(g_j) * u_j)                        (dtype dt, as the 16-bit path)
//   hq, sh: the E4M3 codes and scale of the pair's h row (as xq, sx)
//   eo_c = R(dequant_f(sum_j dec(hq[j]) * dec(Wd8[e,c,j]), sh, sd[e,c]))
// with dequant_f(acc, sa, sw) = acc * sa * sw left to right in fp32; y as in
// oracle_moe_forward. Weights: E4M3 codes [E, D, H] / [E, D, H] / [E, H, D]
// with fp32 row scales [E*D] / [E*D] / [E*H] (oracle_quantize_fp8_rows).
int oracle_moe_forward_w8a8(int dt, const void* x, const uint8_t* wg8, const uint8_t* wu8,
                            const uint8_t* wd8, const float* sg, const float* su, const float* sd,
                            const int32_t* ids, const float* w, int T, int H, int D, int E, int K,
                            const int32_t* tokens, int n_tokens, float* y, float* h_pairs,
                            float* eo_pairs) {
  if (!dtype_ok(dt) || T < 0 || H <= 0 || D <= 0 || E <= 0 || K <= 0) return -1;
  if (!sg || !su || !sd) return -1;
  if (!tokens && n_tokens != T) return -1;
  for (int i = 0; i < n_tokens; ++i) {
    const int t = tokens ? tokens[i] : i;
    if (t < 0 || t >= T) return -1;
    for (int k = 0; k < K; ++k) {
      if (ids[static_cast<int64_t>(t) * K + k] >= E) return -1;
    }
  }
  // E4M3 codes and scale of one row of fp32 values (the per-row quantizer).
  auto quantize_row = [](const float* v, int n, float* codes_as_float) {
    float amax = 0.0f;
    for (int k = 0; k < n; ++k) amax = std::fmax(amax, std::fabs(v[k]));
    const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    for (int k = 0; k < n; ++k) codes_as_float[k] = fp8e4m3_bits_to_float(float_to_fp8e4m3_bits(v[k] / s));
    return s;
  };
#pragma omp parallel
  {
    std::vector<float> xrow(H), xq(H), hbuf(D), hq(D), eo(H), acc(H);
#pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < n_tokens; ++i) {
      const int t = tokens ? tokens[i] : i;
      for (int c = 0; c < H; ++c) xrow[c] = load_elem(dt, x, static_cast<int64_t>(t) * H + c);
      const float sx = quantize_row(xrow.data(), H, xq.data());
      for (int c = 0; c < H; ++c) acc[c] = 0.0f;
      for (int k = 0; k < K; ++k) {
        const int64_t slot = static_cast<int64_t>(t) * K + k;
        const int64_t out_slot = static_cast<int64_t>(i) * K + k;
        const int e = ids[slot];
        if (e < 0) {
          if (h_pairs) for (int j = 0; j < D; ++j) h_pairs[out_slot * D + j] = 0.0f;
          if (eo_pairs) for (int c = 0; c < H; ++c) eo_pairs[out_slot * H + c] = 0.0f;
          continue;
        }
        for (int j = 0; j < D; ++j) {
          const int64_t row = static_cast<int64_t>(e) * D + j;
          float ag = 0.0f, au = 0.0f;
          for (int c = 0; c < H; ++c) {
            ag = std::fma(xq[c], fp8e4m3_bits_to_float(wg8[row * H + c]), ag);
            au = std::fma(xq[c], fp8e4m3_bits_to_float(wu8[row * H + c]), au);
          }
          const float g = ag * sx * sg[row];
          const float u = au * sx * su[row];
          hbuf[j] = round_to(dt, silu(g) * u);
        }
        const float sh = quantize_row(hbuf.data(), D, hq.data());
        for (int c = 0; c < H; ++c) {
          const int64_t row = static_cast<int64_t>(e) * H + c;
          float ad = 0.0f;
          for (int j = 0; j < D; ++j) ad = std::fma(hq[j], fp8e4m3_bits_to_float(wd8[row * D + j]), ad);
          eo[c] = round_to(dt, ad * sh * sd[row]);
        }
        const float wk = w[slot];
        for (int c = 0; c < H; ++c) acc[c] = std::fma(wk, eo[c], acc[c]);
        if (h_pairs) for (int j = 0; j < D; ++j) h_pairs[out_slot * D + j] = hbuf[j];
        if (eo_pairs) for (int c = 0; c < H; ++c) eo_pairs[out_slot * H + c] = eo[c];
      }
      for (int c = 0; c < H; ++c) y[static_cast<int64_t>(i) * H + c] = acc[c];
    }
  }
  return 0;
}

// --------------------------------------------------- MX (block-scaled) ---
// Block-scaled formats ([B] module docstring: the block-scaled mode, MXFP4 /
// MXFP8 through gemm_blockscaled with scale factors SFA / SFB; the formats
// themselves as the OCP Microscaling specification v1.0 defines them):
// along a row, every block of 32 values shares one E8M0 scale X = 2^(e-127)
// (e in [0, 254]); the elements are FP8 E4M3 (max 448) or FP4 E2M1 (values
// 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives). FP4 codes are packed two
// per byte, element 2i in bits 0..3 (sign in bit 3).
//   quantisation of a block with amax = max |v|:  e = floor(log2 amax)
//     - emax_elem + 127 (emax_elem = 8 for E4M3, 2 for E2M1; clamped to
//     [0, 254]; e = 127 for an all-zero block), element = the value nearest
//     to v / X on the element grid (fp32 division; ties to the even code;
//     values beyond the largest magnitude take it).

}  // extern "C"

namespace {

constexpr int kMxBlock = 32;
constexpr int kMxFp8 = 0;   // element format codes (those of the MFMA operand fields)
constexpr int kMxFp4 = 4;

float fp4e2m1_to_float(int c) {
  // sign | 2 exponent bits (bias 1) | 1 mantissa bit; exponent 0 is 0.5 * m
  const int e = (c >> 1) & 3, m = c & 1;
  const float mag = e == 0 ? 0.5f * m : std::ldexp(1.0f + 0.5f * m, e - 1);
  return (c & 8) ? -mag : mag;
}

int float_to_fp4e2m1(float v) {
  const float a = std::fabs(v);
  int best = 0;
  for (int c = 1; c < 8; ++c) {
    const float dc = std::fabs(a - fp4e2m1_to_float(c)), db = std::fabs(a - fp4e2m1_to_float(best));
    if (dc < db || (dc == db && (c & 1) == 0)) best = c;
  }
  return (v < 0.0f && best != 0) ? (best | 8) : best;
}

int mx_scale_exp(float amax, int emax_elem) {
  if (!(amax > 0.0f)) return 127;
  int e2;
  std::frexp(amax, &e2);                    // amax = f * 2^e2, f in [0.5, 1)
  const int e = (e2 - 1) - emax_elem + 127;
  return e < 0 ? 0 : (e > 254 ? 254 : e);
}

float e8m0_to_float(int e) { return std::ldexp(1.0f, e - 127); }

// One row of `cols` values (dtype dt, or fp32 when dt == kF32) to MX codes
// and scales; codes: E4M3 bytes [cols] or packed E2M1 [cols / 2].
void quantize_mx_row(int dt, const void* v, int64_t base, int cols, int fmt, uint8_t* codes,
                     uint8_t* scales) {
  for (int b = 0; b < cols / kMxBlock; ++b) {
    float amax = 0.0f;
    for (int i = 0; i < kMxBlock; ++i) amax = std::fmax(amax, std::fabs(load_elem(dt, v, base + b * kMxBlock + i)));
    const int e = mx_scale_exp(amax, fmt == kMxFp4 ? 2 : 8);
    scales[b] = static_cast<uint8_t>(e);
    const float X = e8m0_to_float(e);
    for (int i = 0; i < kMxBlock; ++i) {
      const int k = b * kMxBlock + i;
      const float q = load_elem(dt, v, base + k) / X;
      if (fmt == kMxFp4) {
        const int c = float_to_fp4e2m1(q);
        if (k % 2 == 0) codes[k / 2] = static_cast<uint8_t>(c);
        else codes[k / 2] = static_cast<uint8_t>(codes[k / 2] | (c << 4));
      } else {
        codes[k] = float_to_fp8e4m3_bits(q);
      }
    }
  }
}

// Decoded value k of an MX row (X * element).
float mx_value(const uint8_t* codes, const uint8_t* scales, int fmt, int64_t k) {
  const float X = e8m0_to_float(scales[k / kMxBlock]);
  const float el = fmt == kMxFp4 ? fp4e2m1_to_float((codes[k >> 1] >> (4 * (k & 1))) & 0xF)
                                 : fp8e4m3_bits_to_float(codes[k]);
  return X * el;
}

}  // namespace

extern "C" {

// MX quantisation of `rows` rows of `cols` values (cols % 32 == 0): fmt 0 =
// MXFP8 (E4M3 codes [rows, cols]), 4 = MXFP4 (packed E2M1 [rows, cols / 2]);
// scales: E8M0 bytes [rows, cols / 32].
int oracle_quantize_mx_rows(int dt, const void* v, int64_t rows, int cols, int fmt,
                            uint8_t* codes, uint8_t* scales) {
  if (!dtype_ok(dt) || rows < 0 || cols <= 0 || cols % kMxBlock || (fmt != kMxFp8 && fmt != kMxFp4)) return -1;
  const int64_t cb = fmt == kMxFp4 ? cols / 2 : cols;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    quantize_mx_row(dt, v, r * cols, cols, fmt, codes + r * cb, scales + r * (cols / kMxBlock));
  }
  return 0;
}

// Decoded MX values (fp32, exact: a power of two times an element value).
int oracle_mx_decode(const uint8_t* codes, const uint8_t* scales, int64_t rows, int cols, int fmt,
                     float* out) {
  if (rows < 0 || cols <= 0 || cols % kMxBlock || (fmt != kMxFp8 && fmt != kMxFp4)) return -1;
  const int64_t cb = fmt == kMxFp4 ? cols / 2 : cols;
  for (int64_t r = 0; r < rows; ++r) {
    for (int k = 0; k < cols; ++k) {
      out[r * cols + k] = mx_value(codes + r * cb, scales + r * (cols / kMxBlock), fmt, k);
    }
  }
  return 0;
}

// The forward with MX experts: MXFP4 weights (packed E2M1 [E, D, H/2] gate /
// up, [E, H, D/2] down, E8M0 scales [E, D, H/32] / [E, H, D/32]) against
// MXFP8 activations: x quantised per token row, h per routed pair. Per pair:
//   g_j  = fp32 fma chain over h ascending of X(x) x(h) * X(wg) wg(h)  (each
//          product of two decoded values is exact), u_j likewise
//   h_j  = R(SiLU(g_j) * u_j)
//   eo_c = R(fp32 fma chain over j of decoded h (MXFP8) * decoded Wd)
// and y as oracle_moe_forward.
int oracle_moe_forward_mx(int dt, const void* x, const uint8_t* wg, const uint8_t* wu,
                          const uint8_t* wd, const uint8_t* sg, const uint8_t* su,
                          const uint8_t* sd, const int32_t* ids, const float* w, int T, int H,
                          int D, int E, int K, const int32_t* tokens, int n_tokens, float* y,
                          float* h_pairs, float* eo_pairs) {
  if (!dtype_ok(dt) || T < 0 || H <= 0 || D <= 0 || E <= 0 || K <= 0 || H % kMxBlock || D % kMxBlock) return -1;
  if (!tokens && n_tokens != T) return -1;
  for (int i = 0; i < n_tokens; ++i) {
    const int t = tokens ? tokens[i] : i;
    if (t < 0 || t >= T) return -1;
    for (int k = 0; k < K; ++k) {
      if (ids[static_cast<int64_t>(t) * K + k] >= E) return -1;
    }
  }
#pragma omp parallel
  {
    std::vector<uint8_t> xc(H), xs(H / kMxBlock), hc(D), hs(D / kMxBlock);
    std::vector<float> xv(H), hv(D), hbuf(D), eo(H), acc(H);
#pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < n_tokens; ++i) {
      const int t = tokens ? tokens[i] : i;
      quantize_mx_row(dt, x, static_cast<int64_t>(t) * H, H, kMxFp8, xc.data(), xs.data());
      for (int c = 0; c < H; ++c) xv[c] = mx_value(xc.data(), xs.data(), kMxFp8, c);
      for (int c = 0; c < H; ++c) acc[c] = 0.0f;
      for (int k = 0; k < K; ++k) {
        const int64_t slot = static_cast<int64_t>(t) * K + k;
        const int64_t out_slot = static_cast<int64_t>(i) * K + k;
        const int e = ids[slot];
        if (e < 0) {
          if (h_pairs) for (int j = 0; j < D; ++j) h_pairs[out_slot * D + j] = 0.0f;
          if (eo_pairs) for (int c = 0; c < H; ++c) eo_pairs[out_slot * H + c] = 0.0f;
          continue;
        }
        for (int j = 0; j < D; ++j) {
          const int64_t row = static_cast<int64_t>(e) * D + j;
          const uint8_t *gc = wg + row * (H / 2), *uc = wu + row * (H / 2);
          const uint8_t *gs = sg + row * (H / kMxBlock), *us = su + row * (H / kMxBlock);
          float g = 0.0f, u = 0.0f;
          for (int c = 0; c < H; ++c) {
            g = std::fma(xv[c], mx_value(gc, gs, kMxFp4, c), g);
            u = std::fma(xv[c], mx_value(uc, us, kMxFp4, c), u);
          }
          hbuf[j] = round_to(dt, silu(g) * u);
        }
        quantize_mx_row(kF32, hbuf.data(), 0, D, kMxFp8, hc.data(), hs.data());
        for (int j = 0; j < D; ++j) hv[j] = mx_value(hc.data(), hs.data(), kMxFp8, j);
        for (int c = 0; c < H; ++c) {
          const int64_t row = static_cast<int64_t>(e) * H + c;
          const uint8_t *dc = wd + row * (D / 2), *ds = sd + row * (D / kMxBlock);
          float o = 0.0f;
          for (int j = 0; j < D; ++j) o = std::fma(hv[j], mx_value(dc, ds, kMxFp4, j), o);
          eo[c] = round_to(dt, o);
        }
        const float wk = w[slot];
        for (int c = 0; c < H; ++c) acc[c] = std::fma(wk, eo[c], acc[c]);
        if (h_pairs) for (int j = 0; j < D; ++j) h_pairs[out_slot * D + j] = hbuf[j];
        if (eo_pairs) for (int c = 0; c < H; ++c) eo_pairs[out_slot * H + c] = eo[c];
      }
      for (int c = 0; c < H; ++c) y[static_cast<int64_t>(i) * H + c] = acc[c];
    }
  }
  return 0;
}

// -------------------------------------------------------- weighted reduce --
// moe_reduce_fused ([C] sections 1-2) and its scaled variants ([C] section 1
// and the commit note on the scaled variants: with_x_sf multiplies once per
// routed slot, with_sf once per output element):
//   y[t, :] = sf[t] * sum over k ascending with pos[t,k] >= 0 of
//             (w[t,k] * x_sf[pos[t,k]]) * X[pos[t,k], :]
// fp32 accumulation with fused multiply-add; w, x_sf, sf == NULL mean ones.
// x_sf is indexed by the expanded row (the row of X), sf by token. X is
// [R, H] in dtype dt (16-bit, fp32 or FP8 E4M3); y is [T, H] fp32 (cast it
// with oracle_from_f32 for a 16-bit or FP8 output). Rows named by masked
// slots are never read. Returns -1 when a position is >= R.
int oracle_reduce_scaled(int dt, const void* X, int64_t R, const int32_t* pos, const float* w,
                         const float* x_sf, const float* sf, int T, int K, int H, float* y) {
  if (!reduce_dtype_ok(dt) || T < 0 || K <= 0 || H <= 0 || R < 0) return -1;
  const int64_t P = static_cast<int64_t>(T) * K;
  for (int64_t s = 0; s < P; ++s) {
    if (pos[s] >= R) return -1;
  }
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    float* yt = y + static_cast<int64_t>(t) * H;
    for (int c = 0; c < H; ++c) yt[c] = 0.0f;
    for (int k = 0; k < K; ++k) {
      const int64_t slot = static_cast<int64_t>(t) * K + k;
      const int32_t p = pos[slot];
      if (p < 0) continue;
      float wk = w ? w[slot] : 1.0f;
      if (x_sf) wk = wk * x_sf[p];
      for (int c = 0; c < H; ++c) {
        yt[c] = std::fma(wk, load_elem(dt, X, static_cast<int64_t>(p) * H + c), yt[c]);
      }
    }
    if (sf) {
      for (int c = 0; c < H; ++c) yt[c] = yt[c] * sf[t];
    }
  }
  return 0;
}

int oracle_reduce(int dt, const void* X, int64_t R, const int32_t* pos, const float* w, int T,
                  int K, int H, float* y) {
  return oracle_reduce_scaled(dt, X, R, pos, w, nullptr, nullptr, T, K, H, y);
}

// ---------------------------------------------------------------- router --
// The gate in front of the routed experts, as the workload recipes of the
// routed-MoE benchmark state it: router weights Wr [E, H] in fp32, scores =
// fp32 softmax of the logits x . Wr^T, the top-k experts by score with ties
// going to the lower expert index, routing weights = the selected scores,
// optionally renormalised to sum to 1 over the k selected experts.
//   logits[t, e] = fp32 fused multiply-add chain over h = 0..H-1 ascending of
//                  x[t, h] * Wr[e, h] (x widened exactly from its dtype), plus
//                  bias[e] in one fp32 addition when a bias is given (the
//                  skewed workload adds 2*log(1/rank) to the logits);
//   selection:     k rounds, each taking the largest remaining logit (the
//                  softmax is strictly increasing, so ranking by logit is
//                  ranking by score), ties to the lower index;
//   scores:        m = the largest logit, Z = sum over e ascending of
//                  expf(logit_e - m), p_e = expf(logit_e - m) / Z;
//   weights:       p of the selected experts in selection order; with
//                  renorm, each divided by their sum (k ascending).
// Inputs must be finite. Writes logits [T, E], ids [T, K], w [T, K].
int oracle_gate(int dt, const void* x, const float* wr, const float* bias, int T, int H, int E,
                int K, int renorm, float* logits, int32_t* ids, float* w) {
  if (!(dt == kF16 || dt == kBF16 || dt == kF32) || T < 0 || H <= 0 || E <= 0 || K <= 0 ||
      K > E) {
    return -1;
  }
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    std::vector<float> xt(H);
    for (int h = 0; h < H; ++h) xt[h] = load_elem(dt, x, static_cast<int64_t>(t) * H + h);
    float* lt = logits + static_cast<int64_t>(t) * E;
    for (int e = 0; e < E; ++e) {
      const float* we = wr + static_cast<int64_t>(e) * H;
      float acc = 0.0f;
      for (int h = 0; h < H; ++h) acc = std::fma(xt[h], we[h], acc);
      lt[e] = bias ? acc + bias[e] : acc;
    }
    std::vector<char> taken(E, 0);
    int32_t* it = ids + static_cast<int64_t>(t) * K;
    for (int k = 0; k < K; ++k) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || lt[e] > lt[best]) best = e;   // strict: ties keep the lower index
      }
      taken[best] = 1;
      it[k] = best;
    }
    const float m = lt[it[0]];
    float z = 0.0f;
    for (int e = 0; e < E; ++e) z += std::exp(lt[e] - m);
    float* wt = w + static_cast<int64_t>(t) * K;
    for (int k = 0; k < K; ++k) wt[k] = std::exp(lt[it[k]] - m) / z;
    if (renorm) {
      float s = 0.0f;
      for (int k = 0; k < K; ++k) s += wt[k];
      for (int k = 0; k < K; ++k) wt[k] = wt[k] / s;
    }
  }
  return 0;
}

}  // extern "C"
