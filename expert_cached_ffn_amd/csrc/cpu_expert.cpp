// ft_cpu_expert_ffn: one expert's SwiGLU FFN on the host CPU, reading the
// expert blob where it lies in host memory -- the CPU side of hybrid miss
// execution (FreeToken 290b model page, "Ejecución híbrida": a cache miss can
// run directly on the CPU instead of being filled over PCIe; the CPU expert
// kernel's effective host bandwidth is the B_h of the miss split).
//
//   y[t] = W_d (silu(W_g x[t]) * (W_u x[t])),   silu(z) = z / (1 + e^-z)
//
// Weights are decoded exactly (every E2M1 value times a power-of-two E8M0
// block scale, and every bf16 weight, is exact in fp32); products of a
// 32-element block are summed in fp32, then scaled; the hidden vector is
// rounded to bf16 before the down projection, as on the GPU.  Each weight
// block is decoded once and applied to every token of the call.  Rows are
// split over a persistent pool of host threads.
//
// Two instruction paths, chosen at run time (ft_cpu_isa): AVX-512 BF16 (FP4
// codes to bf16 by a 16-bit table permute, bf16 pair dot products into fp32;
// the activations stay bf16) and AVX2 + FMA (activations widened to fp32).
#include <immintrin.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <cstdlib>
#include <functional>
#include <memory>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "../../include/ft_moe.h"

namespace ft {
void set_error(const std::string &msg);
void clear_error();
}  // namespace ft

namespace {

// ------------------------------------------------------------------ thread pool

// Workers spin for a short while after a job (decode calls come in bursts a
// fraction of a millisecond apart), then sleep on a condition variable.
class Pool {
 public:
  explicit Pool(int n, int spin_us) : spin_us_(spin_us) {
    for (int i = 0; i < n; ++i) th_.emplace_back([this] { work(); });
  }
  ~Pool() {
    {
      std::lock_guard<std::mutex> g(mu_);
      stop_.store(true);
    }
    cv_.notify_all();
    for (auto &t : th_) t.join();
  }
  int size() const { return int(th_.size()) + 1; }
  // Runs f(0 .. n_tasks-1) on the pool and the calling thread; returns when all
  // are done and no worker is still inside drain(), so the next run() may reset
  // the task counter.  A worker joins a job only while job_ is set (under mu_).
  void run(int n_tasks, const std::function<void(int)> &f) {
    std::lock_guard<std::mutex> one(run_mu_);  // one job at a time
    bool wake;
    {
      std::lock_guard<std::mutex> g(mu_);
      job_ = &f;
      n_ = n_tasks;
      next_.store(0);
      left_.store(n_tasks);
      gen_.fetch_add(1, std::memory_order_release);
      wake = sleepers_ > 0;
    }
    if (wake) cv_.notify_all();
    drain(f, n_tasks);
    while (left_.load(std::memory_order_acquire) > 0) _mm_pause();
    {
      std::lock_guard<std::mutex> g(mu_);
      job_ = nullptr;  // no worker joins from here on
    }
    while (active_.load(std::memory_order_acquire) > 0) _mm_pause();
  }

 private:
  void drain(const std::function<void(int)> &f, int n) {
    for (;;) {
      const int i = next_.fetch_add(1);
      if (i >= n) return;
      f(i);
      left_.fetch_sub(1, std::memory_order_release);
    }
  }
  void work() {
    uint64_t seen = 0;
    for (;;) {
      const auto t0 = std::chrono::steady_clock::now();
      for (int i = 1; gen_.load(std::memory_order_acquire) == seen && !stop_.load(); ++i) {
        _mm_pause();
        if ((i & 255) == 0 && std::chrono::steady_clock::now() - t0 > std::chrono::microseconds(spin_us_)) break;
      }
      const std::function<void(int)> *f;
      int n;
      {
        std::unique_lock<std::mutex> lk(mu_);
        if (!stop_.load() && (gen_.load() == seen || job_ == nullptr)) {
          ++sleepers_;
          cv_.wait(lk, [&] { return stop_.load() || (gen_.load() != seen && job_ != nullptr); });
          --sleepers_;
        }
        if (stop_.load()) return;
        seen = gen_.load();
        f = job_;
        n = n_;
        active_.fetch_add(1);
      }
      drain(*f, n);
      active_.fetch_sub(1, std::memory_order_release);
    }
  }
  const int spin_us_;
  std::vector<std::thread> th_;
  std::mutex mu_, run_mu_;
  std::condition_variable cv_;
  const std::function<void(int)> *job_ = nullptr;  // under mu_
  int n_ = 0;                                      // under mu_
  int sleepers_ = 0;                               // under mu_
  std::atomic<int> next_{0}, left_{0}, active_{0};
  std::atomic<uint64_t> gen_{0};
  std::atomic<bool> stop_{false};
};

int default_threads() {
  if (const char *v = getenv("FTMOE_CPU_THREADS")) {
    const int n = atoi(v);
    if (n > 0) return n;
  }
  const unsigned h = std::thread::hardware_concurrency();
  return h ? int(h) : 1;
}

Pool &pool_for(int threads) {
  static std::mutex mu;
  static std::vector<std::unique_ptr<Pool>> pools;  // one per thread count asked for
  std::lock_guard<std::mutex> g(mu);
  for (auto &p : pools)
    if (p->size() == threads) return *p;
  int spin_us = 300;
  if (const char *v = getenv("FTMOE_CPU_SPIN_US")) spin_us = atoi(v) > 0 ? atoi(v) : 0;
  pools.emplace_back(new Pool(threads - 1, spin_us));
  return *pools.back();
}

// ------------------------------------------------------------------ decoding

inline float bf16_to_f32(uint16_t h) {
  const uint32_t u = uint32_t(h) << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

inline uint16_t f32_to_bf16_bits(float f) {  // nearest even (finite inputs)
  uint32_t b;
  memcpy(&b, &f, 4);
  b += 0x7fffu + ((b >> 16) & 1u);
  return uint16_t(b >> 16);
}

inline float e8m0(uint8_t s) {  // 2^(s - 127) for s in 1..254 (the exponent field itself)
  const uint32_t bits = uint32_t(s) << 23;
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

constexpr int kMaxTok = 8;  // tokens per pass over the weights

// One weight matrix row-major: row r at codes + r * row_bytes (MXFP4: K/2 code
// bytes, element 2j in the low nibble of byte j, and K/32 scale bytes at
// scales + r * (K/32); bf16: K values).
struct Mat {
  const uint8_t *codes;
  const uint8_t *scales;  // MXFP4 only
  int K;
  bool fp4;
};

// ---- AVX2 + FMA path: activations as fp32 -------------------------------------

// Eight FP4 E2M1 codes (element j in bits 4j..4j+3) -> eight floats (unscaled).
inline __m256 e2m1x8(uint32_t word) {
  const __m256 mags = _mm256_setr_ps(0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f);
  const __m256i shifts = _mm256_setr_epi32(0, 4, 8, 12, 16, 20, 24, 28);
  const __m256i v = _mm256_srlv_epi32(_mm256_set1_epi32(int(word)), shifts);
  const __m256i mag = _mm256_and_si256(v, _mm256_set1_epi32(7));
  const __m256i sgn = _mm256_slli_epi32(_mm256_and_si256(v, _mm256_set1_epi32(8)), 28);
  const __m256 m = _mm256_permutevar8x32_ps(mags, mag);
  return _mm256_castsi256_ps(_mm256_xor_si256(_mm256_castps_si256(m), sgn));
}

inline __m256 bf16x8(const uint16_t *p) {
  const __m128i h = _mm_loadu_si128(reinterpret_cast<const __m128i *>(p));
  return _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(h), 16));
}

inline float hsum(__m256 v) {
  const __m128 a = _mm_add_ps(_mm256_castps256_ps128(v), _mm256_extractf128_ps(v, 1));
  const __m128 b = _mm_add_ps(a, _mm_movehl_ps(a, a));
  const __m128 c = _mm_add_ss(b, _mm_shuffle_ps(b, b, 1));
  return _mm_cvtss_f32(c);
}

// out[t] = row r of m . x[t] for nt <= kMaxTok fp32 token rows x[t] (stride ldx).
void dot_avx2(const Mat &m, int r, const float *x, int ldx, int nt, float *out) {
  __m256 acc[kMaxTok];
  for (int t = 0; t < nt; ++t) acc[t] = _mm256_setzero_ps();
  if (m.fp4) {
    const uint8_t *codes = m.codes + size_t(r) * (m.K / 2);
    const uint8_t *scales = m.scales + size_t(r) * (m.K / 32);
    for (int b = 0; b < m.K / 32; ++b) {
      __m256 blk[kMaxTok];
      for (int t = 0; t < nt; ++t) blk[t] = _mm256_setzero_ps();
      for (int g = 0; g < 4; ++g) {
        uint32_t word;
        memcpy(&word, codes + 16 * b + 4 * g, 4);
        const __m256 w = e2m1x8(word);
        const int k0 = b * 32 + g * 8;
        for (int t = 0; t < nt; ++t) blk[t] = _mm256_fmadd_ps(w, _mm256_loadu_ps(x + t * ldx + k0), blk[t]);
      }
      const __m256 s = _mm256_set1_ps(e8m0(scales[b]));
      for (int t = 0; t < nt; ++t) acc[t] = _mm256_fmadd_ps(blk[t], s, acc[t]);
    }
  } else {
    const uint16_t *row = reinterpret_cast<const uint16_t *>(m.codes) + size_t(r) * m.K;
    for (int k = 0; k < m.K; k += 8) {
      const __m256 w = bf16x8(row + k);
      for (int t = 0; t < nt; ++t) acc[t] = _mm256_fmadd_ps(w, _mm256_loadu_ps(x + t * ldx + k), acc[t]);
    }
  }
  for (int t = 0; t < nt; ++t) out[t] = hsum(acc[t]);
}

// ---- AVX-512 BF16 path: activations stay bf16 -----------------------------------
// A 32-element block of FP4 codes becomes 32 bf16 weights with one 16-bit
// table permute (every E2M1 value is exact in bf16); VDPBF16PS then takes the
// block's 32 products (exact in fp32) into 16 fp32 lanes, which are scaled by
// the block's power of two and accumulated.

#define FT_AVX512 __attribute__((target("avx512f,avx512bw,avx512vl,avx512bf16")))

alignas(64) const uint16_t kE2M1Bf16[32] = {
    0x0000, 0x3f00, 0x3f80, 0x3fc0, 0x4000, 0x4040, 0x4080, 0x40c0,   // +0, 0.5, 1, 1.5, 2, 3, 4, 6
    0x8000, 0xbf00, 0xbf80, 0xbfc0, 0xc000, 0xc040, 0xc080, 0xc0c0,   // the same, negative
    0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

FT_AVX512 inline __m512i fp4_block_bf16(const uint8_t *codes, __m512i table) {
  // byte j -> dword j = (low nibble) | (high nibble << 16): words 2j, 2j+1 = elements 2j, 2j+1
  const __m512i t = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i *>(codes)));
  const __m512i idx = _mm512_ternarylogic_epi32(t, _mm512_slli_epi32(t, 12), _mm512_set1_epi32(0x000f000f), 0xa8);
  return _mm512_permutexvar_epi16(idx, table);
}

// out[t] = row r of m . xp[t] for NT bf16 token rows.  CH independent
// accumulator chains per token (blocks b % CH) hide the add latency when few
// tokens share a weight block.
template <int NT>
FT_AVX512 void dot_avx512_n(const Mat &m, int r, const uint16_t *const *xp, float *out) {
  constexpr int CH = NT == 1 ? 4 : (NT == 2 ? 2 : 1);
  __m512 acc[NT][CH];
  for (int t = 0; t < NT; ++t)
    for (int c = 0; c < CH; ++c) acc[t][c] = _mm512_setzero_ps();
  const int nb = m.K / 32;  // a multiple of 4 (K is a multiple of 128)
  if (m.fp4) {
    const __m512i table = _mm512_load_si512(kE2M1Bf16);
    const uint8_t *codes = m.codes + size_t(r) * (m.K / 2);
    const uint8_t *scales = m.scales + size_t(r) * nb;
    alignas(64) float sbuf[16];  // 16 block scales as floats: each block's broadcast is a load
    for (int b0 = 0; b0 < nb; b0 += 16) {
      const int cnt = nb - b0 < 16 ? nb - b0 : 16;  // a multiple of CH
      const __m128i sb = _mm_maskz_loadu_epi8(__mmask16((1u << cnt) - 1u), scales + b0);
      _mm512_store_si512(sbuf, _mm512_slli_epi32(_mm512_cvtepu8_epi32(sb), 23));  // 2^(s-127)
      for (int b1 = 0; b1 < cnt; b1 += CH)
        for (int c = 0; c < CH; ++c) {
          const int b = b0 + b1 + c;
          const __m512i w = fp4_block_bf16(codes + 16 * b, table);
          const __m512 s = _mm512_set1_ps(sbuf[b1 + c]);
          for (int t = 0; t < NT; ++t) {
            const __m512i xv = _mm512_loadu_si512(xp[t] + 32 * b);
            const __m512 blk = _mm512_dpbf16_ps(_mm512_setzero_ps(), (__m512bh)w, (__m512bh)xv);
            acc[t][c] = _mm512_fmadd_ps(blk, s, acc[t][c]);
          }
        }
    }
  } else {
    const uint16_t *row = reinterpret_cast<const uint16_t *>(m.codes) + size_t(r) * m.K;
    for (int b0 = 0; b0 < nb; b0 += CH)
      for (int c = 0; c < CH; ++c) {
        const __m512i w = _mm512_loadu_si512(row + 32 * (b0 + c));
        for (int t = 0; t < NT; ++t)
          acc[t][c] = _mm512_dpbf16_ps(acc[t][c], (__m512bh)w, (__m512bh)_mm512_loadu_si512(xp[t] + 32 * (b0 + c)));
      }
  }
  for (int t = 0; t < NT; ++t) {
    __m512 v = acc[t][0];
    for (int c = 1; c < CH; ++c) v = _mm512_add_ps(v, acc[t][c]);
    out[t] = _mm512_reduce_add_ps(v);
  }
}

FT_AVX512 void dot_avx512(const Mat &m, int r, const uint16_t *const *xp, int nt, float *out) {
  switch (nt) {
    case 1: return dot_avx512_n<1>(m, r, xp, out);
    case 2: return dot_avx512_n<2>(m, r, xp, out);
    case 3: return dot_avx512_n<3>(m, r, xp, out);
    case 4: return dot_avx512_n<4>(m, r, xp, out);
    case 5: return dot_avx512_n<5>(m, r, xp, out);
    case 6: return dot_avx512_n<6>(m, r, xp, out);
    case 7: return dot_avx512_n<7>(m, r, xp, out);
    default: return dot_avx512_n<8>(m, r, xp, out);
  }
}

// ---- ISA selection ---------------------------------------------------------------

int detect_isa() {
  __builtin_cpu_init();
  if (__builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
      __builtin_cpu_supports("avx512vl") && __builtin_cpu_supports("avx512bf16"))
    return FT_CPU_AVX512_BF16;
  if (__builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma")) return FT_CPU_AVX2;
  return 0;
}

std::atomic<int> g_isa{-1};  // in use; -1 = not chosen yet

int active_isa() {
  int v = g_isa.load();
  if (v < 0) {
    v = detect_isa();
    g_isa.store(v);
  }
  return v;
}

struct Expert {
  Mat m[3];  // gate, up, down
  int H, I;
  Expert(const ft_expert_layout *L, const uint8_t *blob) : H(L->H), I(L->I) {
    const bool fp4 = L->wdtype == FT_MXFP4;
    m[0] = Mat{blob + L->off_gate, fp4 ? blob + L->off_sgate : nullptr, L->H, fp4};
    m[1] = Mat{blob + L->off_up, fp4 ? blob + L->off_sup : nullptr, L->H, fp4};
    m[2] = Mat{blob + L->off_down, fp4 ? blob + L->off_sdown : nullptr, L->I, fp4};
  }
};

inline float silu_mul(float g, float u) { return g / (1.0f + std::exp(-g)) * u; }

constexpr int kRowsPerTask = 16;  // enough tasks to balance, a few dozen rows each

// The FFN of one expert for n tokens: bf16 token rows xrow[t], output rows yrow[t].
void expert_ffn(const ft_expert_layout *L, const uint8_t *blob, const uint16_t *const *xrow, int n,
                float *const *yrow, int threads) {
  const Expert ex(L, blob);
  const int H = ex.H, I = ex.I;
  Pool &pool = pool_for(threads);
  const int isa = active_isa();
  for (int t0 = 0; t0 < n; t0 += kMaxTok) {
    const int nt = n - t0 < kMaxTok ? n - t0 : kMaxTok;
    if (isa == FT_CPU_AVX512_BF16) {
      std::vector<uint16_t> h(size_t(nt) * I);  // hidden vectors, bf16
      const uint16_t *hp[kMaxTok];
      for (int t = 0; t < nt; ++t) hp[t] = h.data() + size_t(t) * I;
      const uint16_t *const *xt = xrow + t0;
      pool.run((I + kRowsPerTask - 1) / kRowsPerTask, [&](int task) {
        float g[kMaxTok], u[kMaxTok];
        for (int i = task * kRowsPerTask; i < I && i < (task + 1) * kRowsPerTask; ++i) {
          dot_avx512(ex.m[0], i, xt, nt, g);
          dot_avx512(ex.m[1], i, xt, nt, u);
          for (int t = 0; t < nt; ++t) h[size_t(t) * I + i] = f32_to_bf16_bits(silu_mul(g[t], u[t]));
        }
      });
      pool.run((H + kRowsPerTask - 1) / kRowsPerTask, [&](int task) {
        float o[kMaxTok];
        for (int j = task * kRowsPerTask; j < H && j < (task + 1) * kRowsPerTask; ++j) {
          dot_avx512(ex.m[2], j, hp, nt, o);
          for (int t = 0; t < nt; ++t) yrow[t0 + t][j] = o[t];
        }
      });
    } else {
      std::vector<float> xf(size_t(nt) * H), h(size_t(nt) * I);
      for (int t = 0; t < nt; ++t)
        for (int c = 0; c < H; ++c) xf[size_t(t) * H + c] = bf16_to_f32(xrow[t0 + t][c]);
      pool.run((I + kRowsPerTask - 1) / kRowsPerTask, [&](int task) {
        float g[kMaxTok], u[kMaxTok];
        for (int i = task * kRowsPerTask; i < I && i < (task + 1) * kRowsPerTask; ++i) {
          dot_avx2(ex.m[0], i, xf.data(), H, nt, g);
          dot_avx2(ex.m[1], i, xf.data(), H, nt, u);
          for (int t = 0; t < nt; ++t) h[size_t(t) * I + i] = bf16_to_f32(f32_to_bf16_bits(silu_mul(g[t], u[t])));
        }
      });
      pool.run((H + kRowsPerTask - 1) / kRowsPerTask, [&](int task) {
        float o[kMaxTok];
        for (int j = task * kRowsPerTask; j < H && j < (task + 1) * kRowsPerTask; ++j) {
          dot_avx2(ex.m[2], j, h.data(), I, nt, o);
          for (int t = 0; t < nt; ++t) yrow[t0 + t][j] = o[t];
        }
      });
    }
  }
}

ft_status check_layout(const ft_expert_layout *L, const char *who) {
  if (L == nullptr || L->expert_bytes == 0) {
    ft::set_error(std::string(who) + ": layout not initialised");
    return FT_EINVAL;
  }
  if (L->wdtype != FT_MXFP4 && L->wdtype != FT_BF16) {
    ft::set_error(std::string(who) + ": only bf16 and MXFP4 weights");
    return FT_ENOTSUP;
  }
  if (L->H % 128 != 0 || L->I % 128 != 0) {
    ft::set_error(std::string(who) + ": H and I must be multiples of 128");
    return FT_ENOTSUP;
  }
  return FT_OK;
}

}  // namespace

extern "C" ft_status ft_cpu_expert_ffn(const ft_expert_layout *L, const void *blob, const void *x, int32_t n,
                                       float *y, int32_t n_threads) {
  if (const ft_status st = check_layout(L, "ft_cpu_expert_ffn")) return st;
  if (n < 0 || n_threads < 0) {
    ft::set_error("ft_cpu_expert_ffn: n and n_threads must be non-negative");
    return FT_EINVAL;
  }
  if (n == 0) {
    ft::clear_error();
    return FT_OK;
  }
  if (blob == nullptr || x == nullptr || y == nullptr) {
    ft::set_error("ft_cpu_expert_ffn: NULL pointer argument");
    return FT_EINVAL;
  }
  if (active_isa() == 0) {
    ft::set_error("ft_cpu_expert_ffn: the host CPU has neither AVX2+FMA nor AVX-512 BF16");
    return FT_ENOTSUP;
  }
  const int H = L->H;
  const uint16_t *xb = static_cast<const uint16_t *>(x);
  std::vector<const uint16_t *> xrow(static_cast<size_t>(n));
  std::vector<float *> yrow(static_cast<size_t>(n));
  for (int t = 0; t < n; ++t) {
    xrow[size_t(t)] = xb + size_t(t) * H;
    yrow[size_t(t)] = y + size_t(t) * H;
  }
  expert_ffn(L, static_cast<const uint8_t *>(blob), xrow.data(), n, yrow.data(),
             n_threads > 0 ? n_threads : default_threads());
  ft::clear_error();
  return FT_OK;
}

extern "C" ft_status ft_cpu_miss_rows(const ft_expert_layout *L, const void *bank, int32_t layer, int32_t E,
                                      const int32_t *experts, int32_t n_experts, const int32_t *expert_offsets,
                                      const int32_t *sorted_rows, int32_t T, int32_t k, const void *x,
                                      float *y_rows, int32_t n_threads) {
  if (const ft_status st = check_layout(L, "ft_cpu_miss_rows")) return st;
  if (layer < 0 || E <= 0 || n_experts < 0 || n_experts > E || T < 0 || k <= 0 || n_threads < 0) {
    ft::set_error("ft_cpu_miss_rows: bad sizes");
    return FT_EINVAL;
  }
  if (n_experts == 0 || T == 0) {
    ft::clear_error();
    return FT_OK;
  }
  if (bank == nullptr || experts == nullptr || expert_offsets == nullptr || sorted_rows == nullptr ||
      x == nullptr || y_rows == nullptr) {
    ft::set_error("ft_cpu_miss_rows: NULL pointer argument");
    return FT_EINVAL;
  }
  const int R = T * k;
  if (expert_offsets[0] != 0 || expert_offsets[E] != R) {
    ft::set_error("ft_cpu_miss_rows: expert_offsets must run from 0 to T*k");
    return FT_EINVAL;
  }
  for (int i = 0; i < n_experts; ++i) {
    const int e = experts[i];
    if (e < 0 || e >= E || expert_offsets[e] > expert_offsets[e + 1] || expert_offsets[e + 1] > R) {
      ft::set_error("ft_cpu_miss_rows: expert id or its segment out of range");
      return FT_EINVAL;
    }
    for (int r = expert_offsets[e]; r < expert_offsets[e + 1]; ++r)
      if (sorted_rows[r] < 0 || sorted_rows[r] >= R) {
        ft::set_error("ft_cpu_miss_rows: sorted_rows entry out of range");
        return FT_EINVAL;
      }
  }
  if (active_isa() == 0) {
    ft::set_error("ft_cpu_miss_rows: the host CPU has neither AVX2+FMA nor AVX-512 BF16");
    return FT_ENOTSUP;
  }
  const int H = L->H;
  const int threads = n_threads > 0 ? n_threads : default_threads();
  const uint16_t *xb = static_cast<const uint16_t *>(x);
  const uint8_t *base = static_cast<const uint8_t *>(bank) + (uint64_t(layer) * E) * L->expert_bytes;
  std::vector<const uint16_t *> xrow;
  std::vector<float *> yrow;
  for (int i = 0; i < n_experts; ++i) {
    const int e = experts[i], r0 = expert_offsets[e], n = expert_offsets[e + 1] - r0;
    if (n == 0) continue;
    xrow.resize(size_t(n));
    yrow.resize(size_t(n));
    for (int j = 0; j < n; ++j) {
      xrow[size_t(j)] = xb + size_t(sorted_rows[r0 + j] / k) * H;
      yrow[size_t(j)] = y_rows + size_t(r0 + j) * H;
    }
    expert_ffn(L, base + uint64_t(e) * L->expert_bytes, xrow.data(), n, yrow.data(), threads);
  }
  ft::clear_error();
  return FT_OK;
}

extern "C" ft_status ft_cpu_isa(int32_t request, int32_t *active) {
  const int best = detect_isa();
  if (request == FT_CPU_AVX512_BF16 && best != FT_CPU_AVX512_BF16) {
    ft::set_error("ft_cpu_isa: the host CPU lacks AVX-512 BF16");
    return FT_ENOTSUP;
  }
  if (request == FT_CPU_AVX2 && !(__builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma"))) {
    ft::set_error("ft_cpu_isa: the host CPU lacks AVX2+FMA");
    return FT_ENOTSUP;
  }
  if (request != FT_CPU_ISA_QUERY && request != FT_CPU_ISA_BEST && request != FT_CPU_AVX2 &&
      request != FT_CPU_AVX512_BF16) {
    ft::set_error("ft_cpu_isa: unknown request");
    return FT_EINVAL;
  }
  if (request == FT_CPU_ISA_BEST) g_isa.store(best);
  else if (request != FT_CPU_ISA_QUERY) g_isa.store(request);
  if (active != nullptr) *active = active_isa();
  ft::clear_error();
  return FT_OK;
}
