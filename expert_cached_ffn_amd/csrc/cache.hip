// The GPU expert cache: one LRU over (layer, expert) entries shared by every
// MoE layer, with its slot table updated on the device and misses filled from
// pinned host memory on a side stream.
//
// What the pages fix: GPU memory holds a cache of whole (layer, expert)
// entries while host memory holds the full expert set, the source of truth
// (FreeToken linux page, "Cómo gestiona FreeToken la memoria MoE", memory-tier
// table; FreeToken rtx 4090 page, "Cómo funciona la jerarquía de memoria
// MoE"); one LRU policy is shared across the MoE layers and follows the
// router's recent choices (same sections); hits run on the GPU and misses are
// moved over PCIe from pinned host memory (FreeToken quantization page, "Cómo
// se desplazan los pesos MoE cuantizados por la memoria").
//
// Update order inside one (layer, step), fixed here because the pages do not:
// distinct experts ascending; all hits refreshed first; then each miss takes
// the least recently used slot that holds no member of the step's set (empty
// slots are oldest, lowest index first).
#include <algorithm>
#include <chrono>
#include <vector>

#include "ft_internal.hpp"

namespace ft {

constexpr int kLruThreads = 1024;
constexpr int kFillStreams = 4;  // miss fills spread over this many copy queues (the caller's + 3 own)
constexpr int kLruMaxE = 4096;
constexpr int kLruMaxC = 65536;

enum { LRU_OK = 0, LRU_CAPACITY = 1, LRU_BAD_ID = 2 };

// Written by the LRU kernel into pinned host memory; read by the host after
// the kernel has finished.
struct LruResult {
  int32_t status;
  int32_t n_needed, n_hits, n_misses, n_evictions, n_cpu;
  int32_t pad[2];
  int32_t ev[kLruMaxE][4];  // expert, hit, slot, evicted key (-1 none); ascending expert
};

struct LruState {
  int32_t *map;      // [L*E] key -> slot or -1
  int32_t *owner;    // [C]   slot -> key or -1
  uint64_t *stamp;   // [C]   last use (0 = never)
  uint64_t *clock;   // [1]
  int32_t *protect;  // [E]   keys the last routed step left resident (hits and fills), ascending
  int32_t *n_protect;  // [1]
};

// Device state layout (one allocation): stamps [C] u64, clock (64 B), map
// [L*E] i32, owner [C] i32, protect [E] i32, n_protect (64 B).
inline size_t lru_state_bytes(size_t keys, int C, int E) {
  return size_t(C) * 8 + 64 + keys * 4 + size_t(C) * 4 + size_t(E) * 4 + 64;
}
inline LruState lru_state_at(void *base, size_t keys, int C, int E) {
  uint8_t *p = static_cast<uint8_t *>(base);
  LruState st;
  st.stamp = reinterpret_cast<uint64_t *>(p);
  st.clock = reinterpret_cast<uint64_t *>(p + size_t(C) * 8);
  st.map = reinterpret_cast<int32_t *>(p + size_t(C) * 8 + 64);
  st.owner = st.map + keys;
  st.protect = st.owner + C;
  st.n_protect = st.protect + E;
  return st;
}

__device__ __forceinline__ bool older(uint64_t sa, int a, uint64_t sb, int b) {
  return sa < sb || (sa == sb && a < b);
}

// One workgroup.  Stamps and the slot table are read before any of them is
// written (selection works on the pre-step stamps plus an LDS "taken" bitmap),
// so the kernel never reads its own global writes.
//
// prefetch != 0: a full-layer prefetch (ids = every expert of the layer).  The
// entries the last routed step left resident are taken out of the victim
// choice -- that step's expert FFN may still be reading them (the pages stream
// the next layer in only when the cache has room: FreeToken quantization page,
// "Cómo se desplazan los pesos MoE cuantizados por la memoria") -- and a miss
// that finds no other slot, and every later one, is not prefetched (code 5).
// A routed step records its resident needed keys as the new protected set.
// Number of a step's m misses to fill when the others can run on the host
// CPU: the q in 0..m minimising max(q / b_pcie, (m - q) / b_host), ties to the
// larger q (the miss-split reading of the pages' formula, FreeToken 290b model
// page, "Cómo gestiona FreeToken el prellenado y la decodificación"); b_host
// <= 0: every miss is filled.  Plain double arithmetic, so the decision is the
// same on any IEEE machine.
__device__ inline int miss_split(int m, double b_pcie, double b_host) {
  if (b_host <= 0.0 || m == 0) return m;
  auto t = [&](int q) {
    const double fill = q ? (b_pcie > 0.0 ? double(q) / b_pcie : __builtin_inf()) : 0.0;
    const double cpu = (m - q) ? double(m - q) / b_host : 0.0;
    return fill > cpu ? fill : cpu;
  };
  int best = 0;
  for (int q = 0; q <= m; ++q)
    if (t(q) <= t(best)) best = q;
  return best;
}

__global__ __launch_bounds__(kLruThreads) void lru_step_kernel(LruState st, int layer, const int32_t *__restrict__ ids,
                                                              int R, int E, int C, int prefetch, double b_pcie,
                                                              double b_host,
                                                              int32_t *__restrict__ slot_of_expert,
                                                              int32_t *__restrict__ slot_hits,
                                                              LruResult *__restrict__ res) {
  __shared__ int s_need[kLruMaxE];     // needed flag, then its class: 1 hit, 2 filled, 3 left to the CPU
  __shared__ int s_list[kLruMaxE];     // needed experts, ascending
  __shared__ int s_slot[kLruMaxE];     // slot of needed expert i (hit) or victim (miss)
  __shared__ int s_evk[kLruMaxE];      // evicted key of needed expert i, or -1
  __shared__ uint8_t s_hit[kLruMaxE];  // needed expert i was resident
  __shared__ int s_out[kLruMaxE];      // slot table of the layer after the step
  __shared__ uint32_t s_taken[kLruMaxC / 32];
  __shared__ int s_wcnt[kLruThreads / 64 + 1];
  __shared__ uint64_t s_wst[kLruThreads / 64];
  __shared__ int s_wsl[kLruThreads / 64];
  __shared__ int s_bad, s_n, s_h, s_q, s_full;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NW = kLruThreads / 64;
  const int32_t *lmap = st.map + int64_t(layer) * E;
  if (tid == 0) s_bad = 0;
  for (int e = tid; e < E; e += kLruThreads) {
    s_need[e] = 0;
    s_out[e] = lmap[e];
  }
  for (int w = tid; w < (C + 31) / 32; w += kLruThreads) s_taken[w] = 0u;
  __syncthreads();
  for (int r = tid; r < R; r += kLruThreads) {
    const int e = ids[r];
    if (e < 0 || e >= E) s_bad = 1;
    else s_need[e] = 1;
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0) res->status = LRU_BAD_ID;
    return;
  }
  // Compact the needed set in ascending expert order.
  int base = 0;
  for (int c0 = 0; c0 < E; c0 += kLruThreads) {
    const int e = c0 + tid;
    const bool f = e < E && s_need[e];
    const uint64_t m = __ballot(f);
    if (lane == 0) s_wcnt[wave] = __popcll(m);
    __syncthreads();
    int before = base;
    for (int w = 0; w < wave; ++w) before += s_wcnt[w];
    if (f) s_list[before + __popcll(m & ((uint64_t(1) << lane) - 1))] = e;
    for (int w = 0; w < NW; ++w) base += s_wcnt[w];
    __syncthreads();
  }
  const int n = base;
  if (n > C) {
    if (tid == 0) {
      res->n_needed = n;
      res->status = LRU_CAPACITY;
    }
    return;
  }
  // Phase 1: hits, in list order; hit rank decides the new stamp.
  const uint64_t clk = *st.clock;
  int hbase = 0;
  for (int c0 = 0; c0 < n; c0 += kLruThreads) {
    const int i = c0 + tid;
    int s = -1;
    if (i < n) {
      s = lmap[s_list[i]];
      s_slot[i] = s;
      s_evk[i] = -1;
      s_hit[i] = s >= 0 ? 1 : 0;
      if (s >= 0) atomicOr(&s_taken[s >> 5], 1u << (s & 31));
    }
    const bool hit = i < n && s >= 0;
    const uint64_t m = __ballot(hit);
    if (lane == 0) s_wcnt[wave] = __popcll(m);
    __syncthreads();
    int before = hbase;
    for (int w = 0; w < wave; ++w) before += s_wcnt[w];
    if (hit) st.stamp[s] = clk + uint64_t(before + __popcll(m & ((uint64_t(1) << lane) - 1))) + 1;
    for (int w = 0; w < NW; ++w) hbase += s_wcnt[w];
    __syncthreads();
  }
  const int h = hbase;
  if (prefetch) {  // the last routed step's entries are not victims
    const int np = *st.n_protect;
    for (int i = tid; i < np; i += kLruThreads) {
      const int s = st.map[st.protect[i]];
      if (s >= 0) atomicOr(&s_taken[s >> 5], 1u << (s & 31));
    }
  }
  if (tid == 0) {
    s_q = miss_split(n - h, b_pcie, b_host);
    s_full = 0;
  }
  __syncthreads();
  const int q = s_q;
  // Phase 2: misses in ascending expert order, each of the first q taking the
  // oldest free slot; the others run on the CPU (no slot).
  int mi = 0;
  for (int i = 0; i < n; ++i) {
    if (s_hit[i]) continue;  // uniform across the workgroup
    if (mi >= q || s_full) {  // runs on the CPU / no room for a prefetch: slot and evicted key stay -1
      ++mi;
      continue;
    }
    uint64_t bs = ~uint64_t(0);
    int bsl = 0x7fffffff;
    for (int s = tid; s < C; s += kLruThreads) {
      if (s_taken[s >> 5] & (1u << (s & 31))) continue;
      const uint64_t v = st.stamp[s];
      if (older(v, s, bs, bsl)) {
        bs = v;
        bsl = s;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint64_t ov = __shfl_xor(bs, off);
      const int os = __shfl_xor(bsl, off);
      if (older(ov, os, bs, bsl)) {
        bs = ov;
        bsl = os;
      }
    }
    if (lane == 0) {
      s_wst[wave] = bs;
      s_wsl[wave] = bsl;
    }
    __syncthreads();
    if (tid == 0) {
      uint64_t b = s_wst[0];
      int v = s_wsl[0];
      for (int w = 1; w < NW; ++w)
        if (older(s_wst[w], s_wsl[w], b, v)) {
          b = s_wst[w];
          v = s_wsl[w];
        }
      if (v >= C) {  // every slot is needed or protected (a prefetch only)
        s_full = 1;
      } else {
        s_slot[i] = v;
        s_taken[v >> 5] |= 1u << (v & 31);
        s_evk[i] = st.owner[v];
      }
    }
    __syncthreads();
    ++mi;
  }
  // Apply: stamps of victims, owner / map updates, the layer's slot table.
  __syncthreads();
  int n_evict = 0;
  if (tid == 0) {
    int j = 0, n_cpu = 0, rank = 0, np = 0;
    for (int i = 0; i < n; ++i) {
      const int e = s_list[i];
      const int s = s_slot[i];
      const bool hit = s_hit[i] != 0;
      const bool cpu = !hit && rank++ >= q;  // misses beyond the first q run on the CPU
      const bool noroom = !hit && !cpu && s < 0;  // a prefetch that found no slot
      res->ev[i][0] = e;
      res->ev[i][1] = hit ? 1 : (cpu ? 4 : (noroom ? 5 : 0));
      res->ev[i][2] = s;
      res->ev[i][3] = s_evk[i];
      if (cpu) ++n_cpu;
      s_need[e] = hit ? 1 : (cpu || noroom ? 3 : 2);
      if (!prefetch && !cpu) st.protect[np++] = layer * E + e;
      if (!hit && !cpu && !noroom) {
        st.stamp[s] = clk + uint64_t(h + j) + 1;
        ++j;
        const int ek = s_evk[i];
        if (ek >= 0) {
          st.map[ek] = -1;
          ++n_evict;
          if (ek / E == layer) s_out[ek % E] = -1;
        }
        st.owner[s] = layer * E + e;
        st.map[int64_t(layer) * E + e] = s;
        s_out[e] = s;
      }
    }
    *st.clock = clk + uint64_t(h + j);
    if (!prefetch) *st.n_protect = np;
    res->n_needed = n;
    res->n_hits = h;
    res->n_misses = mi;
    res->n_evictions = n_evict;
    res->n_cpu = n_cpu;
  }
  __syncthreads();
  if (slot_hits == nullptr) {
    for (int e = tid; e < E; e += kLruThreads) slot_of_expert[e] = s_out[e];
  } else {  // split tables: hits now, filled misses after the fills (the other needed experts skipped)
    for (int e = tid; e < E; e += kLruThreads) {
      const int cls = s_need[e];
      slot_hits[e] = cls == 1 ? s_out[e] : (cls ? FT_SLOT_SKIP : -1);
      slot_of_expert[e] = cls == 2 ? s_out[e] : (cls == 1 ? FT_SLOT_SKIP : -1);
    }
  }
  if (tid == 0) {
    __threadfence_system();
    res->status = LRU_OK;
  }
}

}  // namespace ft

using namespace ft;

// Pinned host memory that kernels read and write through its device address.
struct MappedBuf {
  void *host = nullptr;
  void *dev = nullptr;
  size_t bytes = 0;
  ft_status reserve(size_t need) {  // contents are not kept
    if (need <= bytes) return FT_OK;
    release();
    const size_t b = (need + 65535) & ~size_t(65535);
    if (hipHostMalloc(&host, b, hipHostMallocMapped) != hipSuccess) {
      host = nullptr;
      return FT_EHIP;
    }
    if (hipHostGetDevicePointer(&dev, host, 0) != hipSuccess) {
      release();
      return FT_EHIP;
    }
    bytes = b;
    return FT_OK;
  }
  void release() {
    if (host) (void)hipHostFree(host);
    host = dev = nullptr;
    bytes = 0;
  }
};

// Hybrid misses on the host CPU.  The activations and the permutation of a
// step with CPU misses reach host memory through a kernel that writes
// host-mapped memory, and the CPU's rows come back through a kernel that reads
// it: DMA copies on the compute stream would queue behind the step's miss
// fills on the copy engines, and the CPU would first wait for fills it does
// not need.
__global__ void stage_kernel(const uint4 *__restrict__ x, int nx, const int32_t *__restrict__ off, int noff,
                             const int32_t *__restrict__ rows, int nrows, uint4 *hx, int32_t *hoff, int32_t *hrows) {
  const int total = nx + noff + nrows;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    if (i < nx)
      hx[i] = x[i];
    else if (i < nx + noff)
      hoff[i - nx] = off[i - nx];
    else
      hrows[i - nx - noff] = rows[i - nx - noff];
  }
}

// y[list[b]] = hy[list[b]] for workgroup b (rows of H4 float4).
__global__ void patch_kernel(const float4 *__restrict__ hy, const int32_t *__restrict__ list, int H4,
                             float4 *__restrict__ y) {
  const size_t row = size_t(list[blockIdx.x]);
  for (int j = threadIdx.x; j < H4; j += blockDim.x) y[row * H4 + j] = hy[row * H4 + j];
}

struct ft_expert_cache {
  ft_expert_layout L;
  int n_layers, E, C;
  uint8_t *pool;
  const uint8_t *bank;
  hipStream_t copy_stream;
  hipStream_t fill[kFillStreams];   // fill[0] = copy_stream; the others are the cache's own
  hipEvent_t ev_fill[kFillStreams];
  bool pending[kFillStreams];       // a layer prefetch's fills on this queue not yet waited for
  bool unwaited[kFillStreams] = {}; // a split step's fills on this queue (ft_expert_cache_wait_fills)
  int32_t last_filled = 0;          // misses the last step filled
  // a split step launched by ft_expert_cache_plan, waiting for ft_expert_cache_fill
  bool planned = false;
  int32_t plan_layer = 0;
  int32_t *plan_hits = nullptr;
  hipStream_t plan_stream = nullptr;
  int32_t *iota;                    // device [E]: 0..E-1 (the needed set of a layer prefetch)
  double b_pcie = 0.0, b_host = 0.0;  // hybrid split (b_host <= 0: every miss is filled)
  std::vector<int32_t> cpu_list;      // the last step's misses left to the CPU
  int32_t cpu_layer = -1;             // ... and its layer
  // host-mapped buffers of the CPU misses (grown on demand, device address beside)
  uint64_t staged_step = ~uint64_t(0);
  int32_t staged_T = 0, staged_k = 0;
  size_t stage_x_bytes = 0, stage_off_bytes = 0;
  MappedBuf stage, ybuf, list;
  hipEvent_t ev_stage = nullptr, ev_patch = nullptr;
  bool stage_pending = false, patch_pending = false;
  int32_t *pf_slots;                // device [E]: slot table a prefetch writes (unused)
  LruState st;
  void *dev_state;
  LruResult *res_host;   // pinned
  LruResult *res_dev;    // its device address
  hipEvent_t ev_lru, ev_copy;
  int device;
  ft_cache_stats stats;
  // event log: a ring of trace_cap records (0 = off), allocated by ft_expert_cache_set_trace
  std::vector<ft_cache_event> log;
  size_t trace_cap = 0, log_head = 0, log_count = 0;
  std::vector<int32_t> map_mirror;
  // CPU-miss buffers sized by ft_expert_cache_set_split for steps of up to cpu_T tokens x cpu_k picks
  int32_t cpu_T = 0, cpu_k = 0;
};

static void log_event(ft_expert_cache *c, const ft_cache_event &ev) {
  if (c->trace_cap == 0) return;
  c->log[(c->log_head + c->log_count) % c->trace_cap] = ev;
  if (c->log_count < c->trace_cap) {
    ++c->log_count;
  } else {
    c->log_head = (c->log_head + 1) % c->trace_cap;
    ++c->stats.trace_dropped;
  }
}

extern "C" ft_status ft_expert_cache_create(const ft_expert_layout *L, int32_t n_layers, int32_t E,
                                            int32_t capacity, void *slot_pool, const void *host_bank,
                                            hipStream_t copy_stream, ft_expert_cache **out) {
  FT_REQUIRE(out != nullptr, "ft_expert_cache_create: out is NULL");
  *out = nullptr;
  FT_REQUIRE(L != nullptr && L->expert_bytes > 0, "ft_expert_cache_create: layout not initialised");
  FT_REQUIRE(n_layers >= 1 && E >= 1 && capacity >= 1, "ft_expert_cache_create: sizes must be positive");
  FT_SUPPORTED(E <= kLruMaxE, "ft_expert_cache_create: E > 4096");
  FT_SUPPORTED(capacity <= kLruMaxC, "ft_expert_cache_create: capacity > 65536");
  FT_SUPPORTED(int64_t(n_layers) * E <= (int64_t(1) << 20), "ft_expert_cache_create: n_layers*E > 2^20");
  FT_REQUIRE(slot_pool != nullptr && host_bank != nullptr, "ft_expert_cache_create: NULL pool or bank");
  FT_REQUIRE(aligned(slot_pool, 256) && L->expert_bytes % 256 == 0,
             "ft_expert_cache_create: slot_pool must be 256-byte aligned");
  FT_REQUIRE(copy_stream != nullptr, "ft_expert_cache_create: copy_stream must not be the NULL stream");
  hipPointerAttribute_t pa{}, ba{};
  FT_HIP(hipPointerGetAttributes(&pa, slot_pool));
  FT_REQUIRE(pa.type == hipMemoryTypeDevice, "ft_expert_cache_create: slot_pool is not device memory");
  if (hipPointerGetAttributes(&ba, host_bank) != hipSuccess || ba.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return fail(FT_EINVAL, "ft_expert_cache_create: host_bank is not pinned host memory (use hipHostMalloc)");
  }
  int dev = 0;
  FT_HIP(hipGetDevice(&dev));

  ft_expert_cache *c = new ft_expert_cache();
  c->L = *L;
  c->n_layers = n_layers;
  c->E = E;
  c->C = capacity;
  c->pool = static_cast<uint8_t *>(slot_pool);
  c->bank = static_cast<const uint8_t *>(host_bank);
  c->copy_stream = copy_stream;
  c->device = dev;
  const size_t keys = size_t(n_layers) * E;
  const size_t bytes = lru_state_bytes(keys, capacity, E);
  auto cleanup = [&](ft_status st, const std::string &msg) {
    for (int i = 0; i < kFillStreams; ++i) {
      if (i > 0 && c->fill[i]) (void)hipStreamDestroy(c->fill[i]);
      if (c->ev_fill[i]) (void)hipEventDestroy(c->ev_fill[i]);
    }
    if (c->dev_state) (void)hipFree(c->dev_state);
    if (c->iota) (void)hipFree(c->iota);
    if (c->res_host) (void)hipHostFree(c->res_host);
    if (c->ev_lru) (void)hipEventDestroy(c->ev_lru);
    if (c->ev_copy) (void)hipEventDestroy(c->ev_copy);
    delete c;
    return fail(st, msg);
  };
  if (hipMalloc(&c->dev_state, bytes) != hipSuccess) return cleanup(FT_EHIP, "ft_expert_cache_create: hipMalloc failed");
  c->st = lru_state_at(c->dev_state, keys, capacity, E);
  // Empty cache: every key unmapped, every slot free with stamp 0, clock 0, nothing protected.
  if (hipMemset(c->st.map, 0xff, (keys + capacity) * 4) != hipSuccess ||
      hipMemset(c->dev_state, 0, size_t(capacity) * 8 + 64) != hipSuccess ||
      hipMemset(c->st.protect, 0, size_t(E) * 4 + 64) != hipSuccess)
    return cleanup(FT_EHIP, "ft_expert_cache_create: hipMemset failed");
  if (hipHostMalloc(reinterpret_cast<void **>(&c->res_host), sizeof(LruResult), hipHostMallocMapped) != hipSuccess)
    return cleanup(FT_EHIP, "ft_expert_cache_create: hipHostMalloc failed");
  if (hipHostGetDevicePointer(reinterpret_cast<void **>(&c->res_dev), c->res_host, 0) != hipSuccess)
    return cleanup(FT_EHIP, "ft_expert_cache_create: hipHostGetDevicePointer failed");
  if (hipEventCreateWithFlags(&c->ev_lru, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&c->ev_copy, hipEventDisableTiming) != hipSuccess)
    return cleanup(FT_EHIP, "ft_expert_cache_create: hipEventCreate failed");
  c->fill[0] = copy_stream;
  for (int i = 0; i < kFillStreams; ++i) {
    // default priority (the same as every other stream of the library)
    if ((i > 0 && hipStreamCreateWithFlags(&c->fill[i], hipStreamNonBlocking) != hipSuccess) ||
        hipEventCreateWithFlags(&c->ev_fill[i], hipEventDisableTiming) != hipSuccess)
      return cleanup(FT_EHIP, "ft_expert_cache_create: stream or event creation failed");
  }
  if (hipDeviceSynchronize() != hipSuccess) return cleanup(FT_EHIP, "ft_expert_cache_create: sync failed");
  {
    std::vector<int32_t> iota(E);
    for (int e = 0; e < E; ++e) iota[e] = e;
    if (hipMalloc(&c->iota, size_t(E) * 8) != hipSuccess)
      return cleanup(FT_EHIP, "ft_expert_cache_create: hipMalloc failed");
    c->pf_slots = c->iota + E;
    if (hipMemcpy(c->iota, iota.data(), size_t(E) * 4, hipMemcpyHostToDevice) != hipSuccess)
      return cleanup(FT_EHIP, "ft_expert_cache_create: hipMemcpy failed");
  }
  c->stats = ft_cache_stats{};
  c->map_mirror.assign(keys, -1);
  c->cpu_list.reserve(size_t(E));  // a step's CPU misses are at most E: the list never grows past this
  *out = c;
  clear_error();
  return FT_OK;
}

// One LRU update (a step, or a layer prefetch with every expert of the layer
// needed) and its fills.
// A cache step in two halves: cache_launch enqueues the LRU kernel and records
// ev_lru; cache_collect waits for it on the host and acts on its result (the
// event log, the fills, the statistics).  `early`: the compute stream waits
// for a layer prefetch's fills before the LRU kernel rather than after it --
// for a plan, whose caller queues reads of the hit slots before the collect.
static ft_status cache_launch(ft_expert_cache *c, int32_t layer, const int32_t *ids, int R, int32_t *slot_of_expert,
                              int32_t *slot_hits, hipStream_t compute_stream, bool prefetch, bool early) {
  // fills of a split step that the caller did not wait for: order this call's work after them
  for (int q = 0; q < kFillStreams; ++q)
    if (c->unwaited[q]) {
      FT_HIP(hipStreamWaitEvent(compute_stream, c->ev_fill[q], 0));
      c->unwaited[q] = false;
    }
  if (early)
    for (int q = 0; q < kFillStreams; ++q)
      if (c->pending[q]) FT_HIP(hipStreamWaitEvent(compute_stream, c->ev_fill[q], 0));
  c->res_host->status = -1;
  hipLaunchKernelGGL(lru_step_kernel, dim3(1), dim3(kLruThreads), 0, compute_stream, c->st, layer, ids, R, c->E,
                     c->C, prefetch ? 1 : 0, prefetch ? 0.0 : c->b_pcie, prefetch ? 0.0 : c->b_host, slot_of_expert,
                     slot_hits, c->res_dev);
  FT_LAUNCHED("lru_step_kernel");
  FT_HIP(hipEventRecord(c->ev_lru, compute_stream));
  return FT_OK;
}

static ft_status cache_collect(ft_expert_cache *c, int32_t layer, int32_t *slot_hits, hipStream_t compute_stream,
                               bool prefetch, const char *who) {
  FT_HIP(hipEventSynchronize(c->ev_lru));
  const LruResult &r = *c->res_host;
  if (r.status == LRU_BAD_ID) return fail(FT_EINVAL, std::string(who) + ": expert id out of range");
  if (r.status == LRU_CAPACITY)
    return fail(FT_ECAPACITY, std::string(who) + ": " + std::to_string(r.n_needed) + " distinct experts > " +
                                  std::to_string(c->C) + " slots");
  if (r.status != LRU_OK) return fail(FT_EHIP, std::string(who) + ": LRU kernel did not report");
  // Fills that an earlier layer prefetch left in flight come first: the compute
  // stream waits for them (its reads) and so does every queue this call uses
  // (a slot refilled here may be one the prefetch is still writing).
  bool had_pending = false;
  for (int q = 0; q < kFillStreams; ++q) had_pending |= c->pending[q];
  if (had_pending && !prefetch) {
    for (int q = 0; q < kFillStreams; ++q)
      if (c->pending[q]) FT_HIP(hipStreamWaitEvent(compute_stream, c->ev_fill[q], 0));
  }
  const int32_t step = int32_t(c->stats.steps);
  const uint64_t eb = c->L.expert_bytes;
  // Fills go round-robin over kFillStreams copy queues (one queue does not
  // reach the host link's bandwidth).  Each queue first waits for the compute
  // stream up to the LRU kernel: a victim slot may still be read by earlier
  // work enqueued there.
  int fills = 0;
  bool used[kFillStreams] = {};
  if (!prefetch) {
    c->cpu_list.clear();
    c->cpu_layer = layer;
  }
  for (int i = 0; i < r.n_needed; ++i) {
    const int e = r.ev[i][0], code = r.ev[i][1], s = r.ev[i][2], ek = r.ev[i][3];
    const bool hit = code == 1;
    log_event(c, ft_cache_event{step, layer, e, prefetch ? (hit ? 3 : (code == 5 ? 5 : 2)) : code, s, ek});
    if (code == 4) {
      c->cpu_list.push_back(e);  // capacity E reserved at create: no allocation
      continue;
    }
    if (hit || code == 5) continue;
    if (ek >= 0) c->map_mirror[size_t(ek)] = -1;
    c->map_mirror[size_t(layer) * c->E + e] = s;
    const uint8_t *src = c->bank + (uint64_t(layer) * c->E + e) * eb;
    const int q = fills % kFillStreams;
    if (!used[q]) {
      FT_HIP(hipStreamWaitEvent(c->fill[q], c->ev_lru, 0));
      if (had_pending)
        for (int q2 = 0; q2 < kFillStreams; ++q2)
          if (c->pending[q2] && q2 != q) FT_HIP(hipStreamWaitEvent(c->fill[q], c->ev_fill[q2], 0));
      used[q] = true;
    }
    FT_HIP(hipMemcpyAsync(c->pool + uint64_t(s) * eb, src, eb, hipMemcpyHostToDevice, c->fill[q]));
    ++fills;
  }
  if (prefetch) {
    // left in flight; the next step waits for them
    for (int q = 0; q < kFillStreams; ++q)
      if (used[q]) {
        FT_HIP(hipEventRecord(c->ev_fill[q], c->fill[q]));
        c->pending[q] = true;
      }
    c->stats.prefetch_fills += uint64_t(fills);
  } else {
    for (int q = 0; q < kFillStreams; ++q) c->pending[q] = false;  // waited for above
    c->last_filled = fills;
    for (int q = 0; q < kFillStreams; ++q) {
      c->unwaited[q] = false;
      if (!used[q]) continue;
      FT_HIP(hipEventRecord(c->ev_fill[q], c->fill[q]));
      if (slot_hits == nullptr)
        FT_HIP(hipStreamWaitEvent(compute_stream, c->ev_fill[q], 0));
      else
        c->unwaited[q] = true;  // ft_expert_cache_wait_fills
    }
    c->stats.accesses += uint64_t(r.n_needed);
    c->stats.hits += uint64_t(r.n_hits);
    c->stats.misses += uint64_t(r.n_misses);
    c->stats.cpu_misses += uint64_t(r.n_cpu);
    c->stats.steps += 1;
  }
  c->stats.evictions += uint64_t(r.n_evictions);
  c->stats.bytes_h2d += uint64_t(fills) * eb;
  clear_error();
  return FT_OK;
}

static ft_status cache_serve(ft_expert_cache *c, int32_t layer, const int32_t *ids, int R, int32_t *slot_of_expert,
                             int32_t *slot_hits, hipStream_t compute_stream, bool prefetch, const char *who) {
  FT_REQUIRE(!c->planned, std::string(who) + ": a planned step is waiting for ft_expert_cache_fill");
  const ft_status st = cache_launch(c, layer, ids, R, slot_of_expert, slot_hits, compute_stream, prefetch, false);
  if (st != FT_OK) return st;
  return cache_collect(c, layer, slot_hits, compute_stream, prefetch, who);
}

extern "C" ft_status ft_expert_cache_step(ft_expert_cache *c, int32_t layer, const int32_t *topk_ids, int32_t T,
                                          int32_t k, int32_t *slot_of_expert, hipStream_t compute_stream) {
  FT_REQUIRE(c != nullptr, "ft_expert_cache_step: cache is NULL");
  FT_REQUIRE(layer >= 0 && layer < c->n_layers, "ft_expert_cache_step: layer out of range");
  FT_REQUIRE(T >= 0 && k >= 1, "ft_expert_cache_step: need T >= 0, k >= 1");
  FT_REQUIRE(int64_t(T) * k < (int64_t(1) << 31), "ft_expert_cache_step: T*k too large");
  FT_REQUIRE(slot_of_expert != nullptr, "ft_expert_cache_step: slot_of_expert is NULL");
  const int R = T * k;
  FT_REQUIRE(R == 0 || topk_ids != nullptr, "ft_expert_cache_step: topk_ids is NULL");
  return cache_serve(c, layer, topk_ids, R, slot_of_expert, nullptr, compute_stream, false, "ft_expert_cache_step");
}

extern "C" ft_status ft_expert_cache_step_split(ft_expert_cache *c, int32_t layer, const int32_t *topk_ids, int32_t T,
                                                int32_t k, int32_t *slot_hits, int32_t *slot_misses,
                                                int32_t *n_filled, hipStream_t compute_stream) {
  FT_REQUIRE(c != nullptr, "ft_expert_cache_step_split: cache is NULL");
  FT_REQUIRE(layer >= 0 && layer < c->n_layers, "ft_expert_cache_step_split: layer out of range");
  FT_REQUIRE(T >= 0 && k >= 1, "ft_expert_cache_step_split: need T >= 0, k >= 1");
  FT_REQUIRE(int64_t(T) * k < (int64_t(1) << 31), "ft_expert_cache_step_split: T*k too large");
  FT_REQUIRE(slot_hits != nullptr && slot_misses != nullptr && slot_hits != slot_misses,
             "ft_expert_cache_step_split: slot_hits and slot_misses must be two tables");
  const int R = T * k;
  FT_REQUIRE(R == 0 || topk_ids != nullptr, "ft_expert_cache_step_split: topk_ids is NULL");
  const ft_status st =
      cache_serve(c, layer, topk_ids, R, slot_misses, slot_hits, compute_stream, false, "ft_expert_cache_step_split");
  if (st == FT_OK && n_filled != nullptr) *n_filled = c->last_filled;
  return st;
}

extern "C" ft_status ft_expert_cache_plan(ft_expert_cache *c, int32_t layer, const int32_t *topk_ids, int32_t T,
                                          int32_t k, int32_t *slot_hits, int32_t *slot_misses,
                                          hipStream_t compute_stream) {
  FT_REQUIRE(c != nullptr, "ft_expert_cache_plan: cache is NULL");
  FT_REQUIRE(!c->planned, "ft_expert_cache_plan: the previous plan is waiting for ft_expert_cache_fill");
  FT_REQUIRE(layer >= 0 && layer < c->n_layers, "ft_expert_cache_plan: layer out of range");
  FT_REQUIRE(T >= 0 && k >= 1, "ft_expert_cache_plan: need T >= 0, k >= 1");
  FT_REQUIRE(int64_t(T) * k < (int64_t(1) << 31), "ft_expert_cache_plan: T*k too large");
  FT_REQUIRE(slot_hits != nullptr && slot_misses != nullptr && slot_hits != slot_misses,
             "ft_expert_cache_plan: slot_hits and slot_misses must be two tables");
  const int R = T * k;
  FT_REQUIRE(R == 0 || topk_ids != nullptr, "ft_expert_cache_plan: topk_ids is NULL");
  const ft_status st = cache_launch(c, layer, topk_ids, R, slot_misses, slot_hits, compute_stream, false, true);
  if (st != FT_OK) return st;
  c->planned = true;
  c->plan_layer = layer;
  c->plan_hits = slot_hits;
  c->plan_stream = compute_stream;
  clear_error();
  return FT_OK;
}

extern "C" ft_status ft_expert_cache_fill(ft_expert_cache *c, int32_t *n_filled) {
  FT_REQUIRE(c != nullptr, "ft_expert_cache_fill: cache is NULL");
  FT_REQUIRE(c->planned, "ft_expert_cache_fill: no planned step");
  c->planned = false;
  const ft_status st = cache_collect(c, c->plan_layer, c->plan_hits, c->plan_stream, false, "ft_expert_cache_fill");
  if (st == FT_OK && n_filled != nullptr) *n_filled = c->last_filled;
  return st;
}

extern "C" ft_status ft_expert_cache_wait_fills(ft_expert_cache *c, hipStream_t compute_stream) {
  FT_REQUIRE(c != nullptr, "ft_expert_cache_wait_fills: cache is NULL");
  for (int q = 0; q < kFillStreams; ++q)
    if (c->unwaited[q]) {
      FT_HIP(hipStreamWaitEvent(compute_stream, c->ev_fill[q], 0));
      c->unwaited[q] = false;
    }
  clear_error();
  return FT_OK;
}

extern "C" ft_status ft_expert_cache_prefetch_layer(ft_expert_cache *c, int32_t layer, hipStream_t compute_stream) {
  FT_REQUIRE(c != nullptr, "ft_expert_cache_prefetch_layer: cache is NULL");
  FT_REQUIRE(layer >= 0 && layer < c->n_layers, "ft_expert_cache_prefetch_layer: layer out of range");
  return cache_serve(c, layer, c->iota, c->E, c->pf_slots, nullptr, compute_stream, true,
                     "ft_expert_cache_prefetch_layer");
}

extern "C" ft_status ft_expert_cache_set_split(ft_expert_cache *c, double b_pcie, double b_host, int32_t T_max,
                                               int32_t k) {
  FT_REQUIRE(c != nullptr, "ft_expert_cache_set_split: cache is NULL");
  FT_REQUIRE(b_pcie >= 0.0 && b_host >= 0.0 && b_pcie == b_pcie && b_host == b_host,
             "ft_expert_cache_set_split: bandwidths must be non-negative numbers");
  FT_REQUIRE(b_host == 0.0 || b_pcie > 0.0 || b_host > 0.0, "ft_expert_cache_set_split: both bandwidths are zero");
  FT_REQUIRE(!c->planned, "ft_expert_cache_set_split: a planned step is waiting for ft_expert_cache_fill");
  if (b_host > 0.0) {
    FT_REQUIRE(T_max >= 1 && k >= 1 && int64_t(T_max) * k <= (int64_t(1) << 28),
               "ft_expert_cache_set_split: need 1 <= T_max, 1 <= k, T_max*k <= 2^28");
    // the host-mapped buffers of the CPU misses, sized once here (the per-step calls never allocate)
    if (c->stage_pending) FT_HIP(hipEventSynchronize(c->ev_stage));
    if (c->patch_pending) FT_HIP(hipEventSynchronize(c->ev_patch));
    c->stage_pending = c->patch_pending = false;
    const int H = c->L.H;
    const size_t R = size_t(T_max) * k;
    const size_t ob = (size_t(c->E + 1) * 4 + 255) & ~size_t(255);
    if (c->stage.reserve(size_t(T_max) * H * 2 + ob + R * 4) != FT_OK || c->ybuf.reserve(R * H * 4) != FT_OK ||
        c->list.reserve(R * 4) != FT_OK)
      return fail(FT_EHIP, "ft_expert_cache_set_split: hipHostMalloc failed");
    if (c->ev_stage == nullptr) FT_HIP(hipEventCreateWithFlags(&c->ev_stage, hipEventDisableTiming));
    if (c->ev_patch == nullptr) FT_HIP(hipEventCreateWithFlags(&c->ev_patch, hipEventDisableTiming));
    c->cpu_T = T_max;
    c->cpu_k = k;
  }
  c->b_pcie = b_pcie;
  c->b_host = b_host;
  clear_error();
  return FT_OK;
}

extern "C" ft_status ft_expert_cache_set_trace(ft_expert_cache *c, int64_t max_events) {
  FT_REQUIRE(c != nullptr, "ft_expert_cache_set_trace: cache is NULL");
  FT_REQUIRE(max_events >= 0 && max_events <= (int64_t(1) << 28),
             "ft_expert_cache_set_trace: max_events must be in 0..2^28");
  std::vector<ft_cache_event> ring;
  try {
    ring.resize(size_t(max_events));
  } catch (const std::bad_alloc &) {
    return fail(FT_EINVAL, "ft_expert_cache_set_trace: cannot allocate the event ring");
  }
  c->log.swap(ring);
  c->trace_cap = size_t(max_events);
  c->log_head = c->log_count = 0;
  clear_error();
  return FT_OK;
}

extern "C" ft_status ft_expert_cache_cpu_misses(const ft_expert_cache *c, int32_t *experts, int32_t capacity,
                                                int32_t *n) {
  FT_REQUIRE(c != nullptr && n != nullptr, "ft_expert_cache_cpu_misses: NULL argument");
  FT_REQUIRE(capacity >= 0 && (capacity == 0 || experts != nullptr), "ft_expert_cache_cpu_misses: bad buffer");
  *n = int32_t(c->cpu_list.size());
  for (int i = 0; i < *n && i < capacity; ++i) experts[i] = c->cpu_list[size_t(i)];
  clear_error();
  return FT_OK;
}

extern "C" ft_status ft_expert_cache_stage_cpu_misses(ft_expert_cache *c, const void *x, int32_t x_dtype, int32_t T,
                                                      int32_t k, const int32_t *expert_offsets,
                                                      const int32_t *sorted_rows, hipStream_t stream) {
  FT_REQUIRE(c != nullptr, "ft_expert_cache_stage_cpu_misses: cache is NULL");
  FT_REQUIRE(!c->planned, "ft_expert_cache_stage_cpu_misses: a planned step is waiting for ft_expert_cache_fill");
  if (c->cpu_list.empty()) {
    clear_error();
    return FT_OK;
  }
  FT_SUPPORTED(x_dtype == FT_BF16, "ft_expert_cache_stage_cpu_misses: CPU misses take bf16 activations");
  FT_REQUIRE(T >= 1 && k >= 1 && int64_t(T) * k <= (int64_t(1) << 28),
             "ft_expert_cache_stage_cpu_misses: bad T or k");
  FT_REQUIRE(x != nullptr && expert_offsets != nullptr && sorted_rows != nullptr,
             "ft_expert_cache_stage_cpu_misses: NULL pointer argument");
  FT_REQUIRE(aligned(x, 16), "ft_expert_cache_stage_cpu_misses: x must be 16-byte aligned");
  if (T > c->cpu_T || int64_t(T) * k > int64_t(c->cpu_T) * c->cpu_k)
    return fail(FT_ECAPACITY, "ft_expert_cache_stage_cpu_misses: step larger than the T_max x k given to "
                              "ft_expert_cache_set_split");
  const int H = c->L.H, E = c->E, R = T * k;
  const size_t xb = size_t(T) * H * 2;                      // a multiple of 256 (H % 32 == 0)
  const size_t ob = (size_t(E + 1) * 4 + 255) & ~size_t(255);
  // the previous stage's kernel must have written its inputs out before they are replaced
  if (c->stage_pending) FT_HIP(hipEventSynchronize(c->ev_stage));
  const int nx = int(xb / 16), total = nx + (E + 1) + R;
  const int grid = std::min(1024, (total + 255) / 256);
  uint8_t *d = static_cast<uint8_t *>(c->stage.dev);
  hipLaunchKernelGGL(stage_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const uint4 *>(x), nx,
                     expert_offsets, E + 1, sorted_rows, R, reinterpret_cast<uint4 *>(d),
                     reinterpret_cast<int32_t *>(d + xb), reinterpret_cast<int32_t *>(d + xb + ob));
  FT_LAUNCHED("stage_kernel");
  FT_HIP(hipEventRecord(c->ev_stage, stream));
  c->stage_pending = true;
  c->staged_step = c->stats.steps;
  c->staged_T = T;
  c->staged_k = k;
  c->stage_x_bytes = xb;
  c->stage_off_bytes = ob;
  clear_error();
  return FT_OK;
}

extern "C" ft_status ft_expert_cache_run_cpu_misses(ft_expert_cache *c, float *y_rows, hipStream_t stream,
                                                    int32_t n_threads) {
  FT_REQUIRE(c != nullptr, "ft_expert_cache_run_cpu_misses: cache is NULL");
  FT_REQUIRE(!c->planned, "ft_expert_cache_run_cpu_misses: a planned step is waiting for ft_expert_cache_fill");
  if (c->cpu_list.empty()) {
    clear_error();
    return FT_OK;
  }
  FT_REQUIRE(c->stage_pending && c->staged_step == c->stats.steps,
             "ft_expert_cache_run_cpu_misses: call ft_expert_cache_stage_cpu_misses for this step first");
  FT_REQUIRE(y_rows != nullptr && aligned(y_rows, 16), "ft_expert_cache_run_cpu_misses: y_rows NULL or unaligned");
  FT_REQUIRE(n_threads >= 0, "ft_expert_cache_run_cpu_misses: n_threads must be non-negative");
  const int T = c->staged_T, k = c->staged_k, R = T * k, H = c->L.H;
  const auto t0 = std::chrono::steady_clock::now();
  FT_HIP(hipEventSynchronize(c->ev_stage));  // the staged inputs are in host memory
  c->stage_pending = false;
  if (c->patch_pending) FT_HIP(hipEventSynchronize(c->ev_patch));  // the last patch has read ybuf / list
  c->patch_pending = false;
  // ybuf and list hold T*k rows: sized by ft_expert_cache_set_split, checked by the stage call
  const uint8_t *h = static_cast<const uint8_t *>(c->stage.host);
  const int32_t *hoff = reinterpret_cast<const int32_t *>(h + c->stage_x_bytes);
  const int32_t *hrows = reinterpret_cast<const int32_t *>(h + c->stage_x_bytes + c->stage_off_bytes);
  float *hy = static_cast<float *>(c->ybuf.host);
  const ft_status st = ft_cpu_miss_rows(&c->L, c->bank, c->cpu_layer, c->E, c->cpu_list.data(),
                                        int32_t(c->cpu_list.size()), hoff, hrows, T, k, h, hy, n_threads);
  if (st != FT_OK) return st;  // its message is kept
  int32_t *hl = static_cast<int32_t *>(c->list.host);
  int n = 0;
  for (const int32_t e : c->cpu_list)
    for (int r = hoff[e]; r < hoff[e + 1]; ++r) hl[n++] = r;
  if (n > 0) {
    hipLaunchKernelGGL(patch_kernel, dim3(n), dim3(256), 0, stream, static_cast<const float4 *>(c->ybuf.dev),
                       static_cast<const int32_t *>(c->list.dev), H / 4, reinterpret_cast<float4 *>(y_rows));
    FT_LAUNCHED("patch_kernel");
    FT_HIP(hipEventRecord(c->ev_patch, stream));
    c->patch_pending = true;
  }
  c->stats.cpu_ns += uint64_t(
      std::chrono::duration_cast<std::chrono::nanoseconds>(std::chrono::steady_clock::now() - t0).count());
  clear_error();
  return FT_OK;
}

// Resize at a safe point (the pages: the runtime resizes and rebuilds the GPU
// expert cache at safe points of its scheduler when the available GPU memory
// changes; FreeToken quantization page, "Flujo de configuración de la
// cuantización de FreeToken"; FreeToken 290b model page, "Caché elástica").
// Rule (the pages give none): keep the min(new capacity, resident) most
// recently used entries, compacted into slots 0.. in ascending order of their
// old slot (an entry never moves to a higher slot, so the move is safe inside
// one allocation), stamps and clock unchanged, the rest dropped (evictions).
// A rare, host-driven operation: it waits for the cache's streams, reads the
// small state, rebuilds it for the new capacity and copies the kept blobs.
extern "C" ft_status ft_expert_cache_resize(ft_expert_cache *c, int32_t new_capacity, void *new_slot_pool,
                                            hipStream_t stream) {
  FT_REQUIRE(c != nullptr, "ft_expert_cache_resize: cache is NULL");
  FT_REQUIRE(!c->planned, "ft_expert_cache_resize: a planned step is waiting for ft_expert_cache_fill");
  FT_REQUIRE(new_capacity >= 1, "ft_expert_cache_resize: capacity must be positive");
  FT_SUPPORTED(new_capacity <= kLruMaxC, "ft_expert_cache_resize: capacity > 65536");
  FT_REQUIRE(new_slot_pool != nullptr && aligned(new_slot_pool, 256),
             "ft_expert_cache_resize: new_slot_pool must be a 256-byte aligned device buffer");
  hipPointerAttribute_t pa{};
  FT_HIP(hipPointerGetAttributes(&pa, new_slot_pool));
  FT_REQUIRE(pa.type == hipMemoryTypeDevice, "ft_expert_cache_resize: new_slot_pool is not device memory");
  for (int q = 0; q < kFillStreams; ++q) FT_HIP(hipStreamSynchronize(c->fill[q]));
  FT_HIP(hipStreamSynchronize(stream));
  for (int q = 0; q < kFillStreams; ++q) c->pending[q] = c->unwaited[q] = false;  // every fill has landed
  const int C = c->C, C2 = new_capacity;
  const size_t keys = size_t(c->n_layers) * c->E;
  std::vector<uint64_t> stamp(C);
  std::vector<int32_t> owner(C);
  std::vector<int32_t> protect(size_t(c->E) + 16);  // the protected keys and their count (keys stay valid)
  uint64_t clock = 0;
  FT_HIP(hipMemcpy(stamp.data(), c->st.stamp, size_t(C) * 8, hipMemcpyDeviceToHost));
  FT_HIP(hipMemcpy(owner.data(), c->st.owner, size_t(C) * 4, hipMemcpyDeviceToHost));
  FT_HIP(hipMemcpy(&clock, c->st.clock, 8, hipMemcpyDeviceToHost));
  FT_HIP(hipMemcpy(protect.data(), c->st.protect, (size_t(c->E) + 16) * 4, hipMemcpyDeviceToHost));
  // keep the C2 largest stamps among occupied slots (stamps of occupied slots are distinct)
  std::vector<int> used;
  for (int s = 0; s < C; ++s)
    if (owner[s] >= 0) used.push_back(s);
  std::vector<int> by_age(used);
  std::sort(by_age.begin(), by_age.end(), [&](int a, int b) { return stamp[a] > stamp[b]; });
  std::vector<char> keep(C, 0);
  for (size_t i = 0; i < by_age.size() && i < size_t(C2); ++i) keep[by_age[i]] = 1;
  std::vector<uint64_t> stamp2(C2, 0);
  std::vector<int32_t> owner2(C2, -1);
  std::vector<int32_t> map2(keys, -1);
  uint8_t *pool2 = static_cast<uint8_t *>(new_slot_pool);
  const uint64_t eb = c->L.expert_bytes;
  int nxt = 0;
  uint64_t dropped = 0;
  for (int s : used) {  // ascending old slot
    if (!keep[s]) {
      ++dropped;
      continue;
    }
    owner2[nxt] = owner[s];
    stamp2[nxt] = stamp[s];
    map2[size_t(owner[s])] = nxt;
    if (pool2 != c->pool || nxt != s)
      FT_HIP(hipMemcpyAsync(pool2 + uint64_t(nxt) * eb, c->pool + uint64_t(s) * eb, eb, hipMemcpyDeviceToDevice,
                            stream));
    ++nxt;
  }
  // new device state for the new capacity (same layout as at creation)
  void *state2 = nullptr;
  FT_HIP(hipMalloc(&state2, lru_state_bytes(keys, C2, c->E)));
  const LruState st2 = lru_state_at(state2, keys, C2, c->E);
  hipError_t e = hipMemcpy(st2.stamp, stamp2.data(), size_t(C2) * 8, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(st2.clock, &clock, 8, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(st2.map, map2.data(), keys * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(st2.owner, owner2.data(), size_t(C2) * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(st2.protect, protect.data(), (size_t(c->E) + 16) * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    (void)hipFree(state2);
    return fail(FT_EHIP, std::string("ft_expert_cache_resize: ") + hipGetErrorString(e));
  }
  (void)hipFree(c->dev_state);
  c->dev_state = state2;
  c->st = st2;
  c->C = C2;
  c->pool = pool2;
  c->map_mirror = map2;
  c->stats.evictions += dropped;
  clear_error();
  return FT_OK;
}

extern "C" ft_status ft_expert_cache_stats(const ft_expert_cache *c, ft_cache_stats *out) {
  FT_REQUIRE(c != nullptr && out != nullptr, "ft_expert_cache_stats: NULL argument");
  *out = c->stats;
  clear_error();
  return FT_OK;
}

extern "C" ft_status ft_expert_cache_trace(const ft_expert_cache *c, void *host_buf, size_t bytes, size_t *needed) {
  FT_REQUIRE(c != nullptr, "ft_expert_cache_trace: cache is NULL");
  const size_t all = c->log_count * sizeof(ft_cache_event);
  if (needed) *needed = all;
  if (host_buf != nullptr && bytes > 0) {
    const size_t n = std::min(c->log_count, bytes / sizeof(ft_cache_event));
    ft_cache_event *out = static_cast<ft_cache_event *>(host_buf);
    for (size_t i = 0; i < n; ++i) out[i] = c->log[(c->log_head + i) % c->trace_cap];
  }
  clear_error();
  return FT_OK;
}

extern "C" ft_status ft_expert_cache_lookup(const ft_expert_cache *c, int32_t layer, int32_t expert, int32_t *slot) {
  FT_REQUIRE(c != nullptr && slot != nullptr, "ft_expert_cache_lookup: NULL argument");
  FT_REQUIRE(layer >= 0 && layer < c->n_layers && expert >= 0 && expert < c->E,
             "ft_expert_cache_lookup: layer or expert out of range");
  *slot = c->map_mirror[size_t(layer) * c->E + expert];
  clear_error();
  return FT_OK;
}

extern "C" ft_status ft_expert_cache_destroy(ft_expert_cache *c) {
  if (c == nullptr) {
    clear_error();
    return FT_OK;
  }
  hipError_t e1 = hipSuccess;
  for (int q = 0; q < kFillStreams; ++q) {
    const hipError_t eq = hipStreamSynchronize(c->fill[q]);
    if (e1 == hipSuccess) e1 = eq;
    if (q > 0) (void)hipStreamDestroy(c->fill[q]);
    (void)hipEventDestroy(c->ev_fill[q]);
  }
  if (c->ev_stage) {
    (void)hipEventSynchronize(c->ev_stage);
    (void)hipEventDestroy(c->ev_stage);
  }
  if (c->ev_patch) {
    (void)hipEventSynchronize(c->ev_patch);
    (void)hipEventDestroy(c->ev_patch);
  }
  c->stage.release();
  c->ybuf.release();
  c->list.release();
  (void)hipFree(c->dev_state);
  (void)hipFree(c->iota);
  (void)hipHostFree(c->res_host);
  (void)hipEventDestroy(c->ev_lru);
  (void)hipEventDestroy(c->ev_copy);
  delete c;
  if (e1 != hipSuccess) return fail(FT_EHIP, std::string("ft_expert_cache_destroy: ") + hipGetErrorString(e1));
  clear_error();
  return FT_OK;
}
