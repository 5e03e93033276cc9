// Error text, version, expert blob layout and workspace sizing.
#include "ft_internal.hpp"


namespace ft {

static thread_local std::string g_last_error;

void set_error(const std::string &msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }

}  // namespace ft

static uint64_t round_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

extern "C" const char *ft_last_error(void) { return ft::g_last_error.c_str(); }

extern "C" const char *ft_version(void) { return "ftmoe 0.1 gfx950"; }

// One expert = one contiguous blob; the same layout in a GPU slot and in the
// pinned host bank, so a miss fill is one straight copy (FreeToken rtx 4090
// page, "Cómo funciona la jerarquía de memoria MoE": a whole (layer, expert)
// entry under one mapping on both sides).
extern "C" ft_status ft_expert_layout_init(int32_t wdtype, int32_t H, int32_t I,
                                           ft_expert_layout *out) {
  FT_REQUIRE(out != nullptr, "ft_expert_layout_init: out is NULL");
  FT_REQUIRE(H >= 1 && I >= 1, "ft_expert_layout_init: H and I must be positive");
  FT_REQUIRE(uint64_t(H) * uint64_t(I) <= (uint64_t(1) << 36), "ft_expert_layout_init: expert too large");
  ft_expert_layout L = {};
  L.wdtype = wdtype;
  L.H = H;
  L.I = I;
  const uint64_t n = uint64_t(H) * uint64_t(I);
  uint64_t pos = 0;
  auto place = [&](uint64_t bytes) {
    uint64_t at = round_up(pos, 256);
    pos = at + bytes;
    return at;
  };
  switch (wdtype) {
    case FT_F32:
    case FT_BF16: {
      const uint64_t es = wdtype == FT_F32 ? 4 : 2;
      L.off_gate = place(n * es);
      L.off_up = place(n * es);
      L.off_down = place(n * es);
      break;
    }
    case FT_MXFP4:
      FT_REQUIRE(H % 32 == 0 && I % 32 == 0,
                 "ft_expert_layout_init: MXFP4 needs H and I multiples of 32");
      L.off_gate = place(n / 2);
      L.off_up = place(n / 2);
      L.off_down = place(n / 2);
      L.off_sgate = place(n / 32);
      L.off_sup = place(n / 32);
      L.off_sdown = place(n / 32);
      break;
    case FT_NVFP4:
      FT_REQUIRE(H % 16 == 0 && I % 16 == 0,
                 "ft_expert_layout_init: NVFP4 needs H and I multiples of 16");
      L.off_gate = place(n / 2);
      L.off_up = place(n / 2);
      L.off_down = place(n / 2);
      L.off_sgate = place(n / 16);
      L.off_sup = place(n / 16);
      L.off_sdown = place(n / 16);
      L.off_tscale = place(3 * 4);
      break;
    default:
      return ft::fail(FT_EINVAL, "ft_expert_layout_init: unknown weight dtype");
  }
  L.expert_bytes = round_up(pos, 4096);
  *out = L;
  ft::clear_error();
  return FT_OK;
}

extern "C" size_t ft_workspace_bytes(int32_t which, int32_t T, int32_t k, int32_t E, int32_t H,
                                     int32_t I) {
  if (T < 0 || k < 0 || E < 0 || H < 0 || I < 0) return 0;
  switch (which) {
    case FT_WS_PERMUTE:
      return ft::permute_workspace_bytes(T, k, E);
    case FT_WS_FFN:
      return ft::ffn_workspace_bytes(T, k, E, H, I);
    case FT_WS_ROUTE_PERMUTE:
      return ft::permute_workspace_bytes(T, k, E);
    case FT_WS_LAYER: {  // the one-token kernel's wait words, then the permutation's counts or the FFN's rows
      const size_t a = ft::permute_workspace_bytes(T, k, E), b = ft::ffn_workspace_bytes(T, k, E, H, I);
      return ft::kLayerWaitBytes + (a > b ? a : b);
    }
    default:
      return 0;
  }
}
