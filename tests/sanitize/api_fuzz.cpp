// api_fuzz.cpp -- host-only harness for the C ABI's argument handling under
// AddressSanitizer / UndefinedBehaviorSanitizer (built with g++ by
// tests/test_sanitizers.py; no device code).  The launchers are stubs that
// check what attn_api.cpp hands them: every layout it resolves must keep
// one head's rows, and the rows a tile copy reads past the end, inside a
// 32-bit byte range, and every pointer must be the caller's.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>

#include "attn.h"
#include "attn_internal.h"

namespace {
int g_launches = 0;
bool layout_ok(const attn::Layout& l, int n, int d) {
  if (l.sb < 0 || l.sh < 0 || l.sn < d) return false;
  return (double)(n + 256) * l.sn * 2.0 < 2147483648.0;
}
void check(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "stub launcher: %s\n", what);
    std::abort();
  }
}
}  // namespace

namespace attn {
hipError_t launch_fwd(const FwdArgs& a, int d, bool, int guard, bool, int pv, hipStream_t) {
  ++g_launches;
  check(a.q && a.k && a.v && a.o && a.row_m && a.row_l && a.row_flags, "null pointer");
  check(a.Hq % a.Hkv == 0 && a.group == a.Hq / a.Hkv, "group");
  check(guard >= 0 && guard <= 2 && pv >= 0 && pv <= 2 && (d == 64 || d == 128), "mode");
  for (const Layout* l : {&a.lq, &a.lk, &a.lv, &a.lo}) check(layout_ok(*l, a.N, d), "layout");
  return hipSuccess;
}
hipError_t launch_fwd_block(const FwdArgs& a, int d, bool, int, bool, bool, hipStream_t) {
  ++g_launches;
  for (const Layout* l : {&a.lq, &a.lk, &a.lv, &a.lo}) check(layout_ok(*l, a.N, d), "layout");
  return hipSuccess;
}
hipError_t launch_bwd_dkdv(const BwdArgs& a, int d, bool, hipStream_t) {
  ++g_launches;
  check(a.q && a.k && a.v && a.dout && a.row_m && a.row_l && a.delta && a.dk && a.dv, "null pointer");
  for (const Layout* l : {&a.lq, &a.lk, &a.lv, &a.ldo, &a.ldk, &a.ldv}) check(layout_ok(*l, a.N, d), "layout");
  return hipSuccess;
}
hipError_t launch_bwd_dq(const BwdArgs& a, int d, bool, bool delta_dp, hipStream_t) {
  ++g_launches;
  check(a.q && a.k && a.v && a.dout && a.row_m && a.row_l && a.delta && a.dq, "null pointer");
  check(delta_dp || a.o, "O needed for rowsum(dO*O)");
  for (const Layout* l : {&a.lq, &a.lk, &a.lv, &a.ldo, &a.ldq}) check(layout_ok(*l, a.N, d), "layout");
  return hipSuccess;
}
}  // namespace attn

int main() {
  std::mt19937_64 rng(12345);
  auto pick = [&](std::initializer_list<long long> v) { return *(v.begin() + rng() % v.size()); };
  alignas(16) static char buf[4096];
  void* P = buf;
  int ok = 0, refused = 0;
  for (int it = 0; it < 200000; ++it) {
    attn_params p;
    std::memset(&p, 0, sizeof p);
    p.batch = (int)pick({-1, 0, 1, 2, 7, 1 << 16});
    p.heads_kv = (int)pick({0, 1, 2, 3, 8});
    p.heads_q = p.heads_kv * (int)pick({1, 2, 4}) + (int)pick({0, 0, 0, 1});
    p.seqlen = (int)pick({-5, 0, 1, 63, 128, 1000, 8192, 1 << 20, 1 << 24});
    p.head_dim = (int)pick({0, 32, 64, 96, 128});
    p.softmax_scale = (float)pick({0, 0, 1, -1}) * 0.125f;
    if (rng() % 50 == 0) p.softmax_scale = NAN;
    p.beta = (float)pick({0, 1, 2, 8});
    p.tie_eps = (float)pick({-1, 0, 1}) * 1e-3f;
    p.shift_eps = (float)pick({0, 1}) * 0.03125f;
    p.flags = (uint32_t)(rng() & 0x7ff);
    attn_strides* st[] = {&p.q_stride, &p.k_stride, &p.v_stride, &p.o_stride,
                          &p.do_stride, &p.dq_stride, &p.dk_stride, &p.dv_stride};
    if (rng() % 2) {
      // a valid call (dense or fused-QKV strides), then at most one field
      // moved to a random value
      p.batch = 2;
      p.heads_kv = (int)pick({1, 2, 4});
      p.heads_q = 4;
      p.seqlen = (int)pick({1, 100, 1000, 4096});
      p.head_dim = (int)pick({64, 128});
      p.beta = 2.0f;
      p.tie_eps = 1e-3f;
      p.shift_eps = 0.03125f;
      p.flags = (uint32_t)pick({0x0, 0x1, 0x3, 0x5, 0x9, 0x13, 0x23, 0x41, 0x81, 0x181, 0x201, 0x601});
      const bool fused = rng() % 2;
      for (int t = 0; t < 8; ++t) {
        const int h = (t == 1 || t == 2 || t == 6 || t == 7) ? p.heads_kv : p.heads_q;
        if (fused) *st[t] = {(int64_t)p.seqlen * 3 * 4 * p.head_dim, p.head_dim, 3LL * 4 * p.head_dim};
        else *st[t] = {0, 0, 0};
        (void)h;
      }
      switch (rng() % 8) {
        case 0: st[rng() % 8]->row = pick({0, 8, 60, 1LL << 33}); break;
        case 1: st[rng() % 8]->head = pick({-8, 4, 1LL << 40}); break;
        case 2: p.flags = (uint32_t)(rng() & 0x7ff); break;
        case 3: p.seqlen = (int)pick({0, 1 << 24}); break;
        default: break;
      }
    } else {
      for (attn_strides* s : st) {
        if (rng() % 3 == 0) {
          s->batch = pick({-8, 0, 8, 1 << 20, 1LL << 40});
          s->head = pick({0, 4, 64, 128, 1 << 16, 1LL << 36});
          s->row = pick({0, 8, 60, 64, 128, 2304, 1 << 20, 1LL << 33});
        }
      }
    }
    void* ptr[14];
    for (void*& x : ptr) x = (rng() % 40 == 0) ? nullptr : (rng() % 40 == 0 ? (void*)(buf + 8) : P);
    int32_t bm, bn, rn, ch, bb, pc;
    int rc = attn_schedule(&p, &bm, &bn, &rn, &ch, &bb, &pc);
    // the workspace query agrees with the parameter checks
    if ((attn_bwd_workspace_bytes(&p) == 0) != (rc == 0)) std::abort();
    rc |= attn_fwd(&p, ptr[0], ptr[1], ptr[2], ptr[3], (float*)ptr[4], (float*)ptr[5], (uint8_t*)ptr[6],
                   rng() % 2 ? ptr[7] : nullptr, rng() % 2 ? (float*)ptr[8] : nullptr, nullptr);
    rc |= attn_bwd(&p, ptr[0], ptr[1], ptr[2], ptr[3], ptr[4], (const float*)ptr[5], (const float*)ptr[6],
                   ptr[7], ptr[8], ptr[9], (float*)ptr[10], rng() % 2 ? (float*)ptr[11] : nullptr, nullptr);
    if (rc) ++refused; else ++ok;
    if (attn_strerror(rc % 8)[0] == '\0') std::abort();
  }
  std::printf("api fuzz: %d accepted, %d refused, %d stub launches\n", ok, refused, g_launches);
  return 0;
}
