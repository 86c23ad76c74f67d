// Host-side check of the QMoE contract validator and launch planner
// (csrc/qmoe_plan.cpp), built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_plan_sanitizers.py.
//
// A seeded generator draws tensor descriptors and attributes around the
// operator's contract (QMoE WebGPU manifest: inputs, attributes,
// attributeConstraints, derive.quantShapeOk / quantScalesOk /
// quantBlockSizeOk / quantContract): valid shapes of every scale layout and
// bit width, one-GPU expert shares, and mutations of one field at a time
// (ranks 0..4, negative, zero and huge extents, wrong dtypes, attribute
// values outside their sets).  Every validation runs under the sanitizers;
// for every accepted case the plan must satisfy its own invariants:
//   - workspace regions 256-byte aligned, inside the total, not overlapping;
//   - room for the tile table (the most tiles routing can produce) and for
//     every intermediate at its stated size;
//   - the streaming split of each GEMM tiles its reduction exactly.
// Exit status 0 when every invariant held; a sanitizer report aborts.
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "qmoe.h"
#include "qmoe_plan.h"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t next() {  // splitmix64
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
int64_t pick(const std::vector<int64_t>& v) { return v[next() % v.size()]; }

int failures = 0;
#define EXPECT(cond, ...)                                   \
  do {                                                      \
    if (!(cond)) {                                          \
      ++failures;                                           \
      std::fprintf(stderr, "invariant failed: %s: ", #cond); \
      std::fprintf(stderr, __VA_ARGS__);                    \
      std::fprintf(stderr, "\n");                           \
    }                                                       \
  } while (0)

qmoe_tensor tensor(int32_t dtype, int32_t rank, int64_t d0, int64_t d1 = 0, int64_t d2 = 0) {
  qmoe_tensor t;
  std::memset(&t, 0, sizeof t);
  t.data = nullptr;
  t.dtype = dtype;
  t.rank = rank;
  t.dims[0] = d0;
  t.dims[1] = d1;
  t.dims[2] = d2;
  return t;
}

struct Case {
  qmoe_tensor in, router, w1, s1, w2, s2, out;
  qmoe_attrs a;
};

Case valid_case() {
  Case c;
  qmoe_attrs_default(&c.a);
  const int bits = next() % 2 ? 4 : 8;
  const bool swiglu = next() % 2;
  const int64_t bs = pick({0, 0, 16, 32, 64, 128, 256});
  const int64_t unit = bs ? bs : (bits == 4 ? 2 : 1);
  const int64_t H = unit * pick({1, 2, 3, 4, 7, 16, 64});
  const int64_t I = pick({0, 1, 1, 2, 5, 8, 56}) * unit;
  const int64_t E = pick({1, 2, 4, 8, 64, 128, 1024});
  const int64_t T = pick({0, 1, 7, 16, 17, 64, 65, 200, 1024, 1025, 8192});
  const int64_t k = 1 + (int64_t)(next() % (uint64_t)std::min<int64_t>(E, 8));
  // one-GPU share: the weights hold El experts from first
  int64_t El = E, first = 0;
  if (next() % 3 == 0) {
    El = (int64_t)(next() % (uint64_t)(E + 1));
    first = (int64_t)(next() % (uint64_t)(E - El + 1));
  }
  const int64_t F = (swiglu ? 2 : 1) * I;
  const int64_t pack = bits == 4 ? 2 : 1;
  c.a.k = (int32_t)k;
  c.a.expert_weight_bits = bits;
  c.a.block_size = (int32_t)bs;
  c.a.activation_type = swiglu ? QMOE_ACT_SWIGLU : QMOE_ACT_RELU;
  c.a.swiglu_fusion = swiglu ? 1 : 0;
  c.a.routing = next() % 2 ? QMOE_ROUTE_MOE : QMOE_ROUTE_QMOE;
  c.a.normalize_routing_weights = (int32_t)(next() % 2);
  c.a.first_expert = (int32_t)first;
  if (swiglu && next() % 2) {
    c.a.has_swiglu_limit = 1;
    c.a.swiglu_limit = 7.f;
  }
  if (next() % 2) {
    c.in = tensor(QMOE_F32, 2, T, H);
  } else {
    const int64_t B = T % 2 == 0 && T > 0 ? 2 : 1;
    c.in = tensor(QMOE_F32, 3, B, T / B, H);
  }
  c.router = tensor(QMOE_F32, 2, T, E);
  c.w1 = tensor(QMOE_U8, 3, El, F, H / pack);
  c.w2 = tensor(QMOE_U8, 3, El, H, I / pack);
  c.s1 = bs ? tensor(QMOE_F32, 3, El, F, H / bs) : tensor(QMOE_F32, 2, El, F);
  c.s2 = bs ? tensor(QMOE_F32, 3, El, H, I / bs) : tensor(QMOE_F32, 2, El, H);
  c.out = c.in;
  return c;
}

void mutate(Case& c) {
  qmoe_tensor* ts[] = {&c.in, &c.router, &c.w1, &c.s1, &c.w2, &c.s2, &c.out};
  switch (next() % 8) {
    case 0: {  // one extent
      qmoe_tensor* t = ts[next() % 7];
      t->dims[next() % 3] = pick({-1, 0, 1, 3, (int64_t)1 << 40, INT64_C(-9223372036854775807)});
      break;
    }
    case 1:
      ts[next() % 7]->rank = (int32_t)(next() % 5);
      break;
    case 2:
      ts[next() % 7]->dtype = (int32_t)(next() % 9);
      break;
    case 3:
      c.a.k = (int32_t)pick({-1, 0, 1, 2, 9, 1025, 2147483647});
      break;
    case 4:
      c.a.block_size = (int32_t)pick({-64, 1, 8, 24, 48, 4096});
      break;
    case 5:
      c.a.first_expert = (int32_t)pick({-1, 1, 7, 1024, 2147483647});
      break;
    case 6:
      c.a.expert_weight_bits = (int32_t)pick({0, 2, 3, 16});
      break;
    default:
      c.a.activation_type = (int32_t)pick({-1, 2, 9});
      c.a.swiglu_fusion = (int32_t)pick({0, 1, 2, 3});
      break;
  }
}

void check_plan(const qmoe::Dims& d, const qmoe::Plan& p) {
  using qmoe::Plan;
  struct Region {
    size_t off, len;
    const char* name;
  };
  const int64_t S = p.S;
  const int64_t groups = p.share ? d.El + 1 : d.E;
  const size_t stream_part = p.s1.on && p.s1.splits > 1 ? sizeof(float) * p.s1.splits * S * d.F : 0;
  const std::vector<Region> rs = {
      {p.off_topk_idx, 4 * (size_t)S, "topk_idx"},
      {p.off_topk_w, 4 * (size_t)S, "topk_w"},
      {p.off_counts, 4 * (size_t)groups, "counts"},
      {p.off_offsets, 4 * (size_t)(groups + 1), "offsets"},
      {p.off_perm, 4 * (size_t)S, "perm"},
      {p.off_tiles, 16 * (size_t)p.max_tiles, "tiles"},
      {p.off_ntiles, 16, "ntiles"},
      {p.off_hist, 4 * (size_t)(p.nchunks * groups), "hist"},
      {p.off_xa, p.s1.on ? 0 : 4 * (size_t)(d.T * p.kp1), "xa"},
      {p.off_act, 4 * (size_t)(S * p.kp2), "act"},
      {p.off_exp1, 4 * (size_t)d.T, "exp1"},
      {p.off_exp2, 4 * (size_t)S, "exp2"},
      {p.off_seg, 4 * (size_t)p.max_tiles * p.seg_n, "seg"},
      {p.off_segrows, 4 * (size_t)S * p.seg_n, "segrows"},
      {p.off_segflag, p.seg_n > 0 ? (size_t)4 : 0, "segflag"},
      {p.off_slot, d.I > 0 ? sizeof(float) * p.splits2 * S * d.H : 0, "slot"},
      {p.off_part1, stream_part, "part1"},
      {p.off_trows, p.s1.on || p.s2.on ? 4 * (size_t)(p.max_tiles * p.bm) : 0, "trows"},
      {p.off_local, p.share ? 4 * (size_t)S : 0, "local"},
  };
  for (size_t i = 0; i < rs.size(); ++i) {
    EXPECT(rs[i].off % 256 == 0, "%s at %zu", rs[i].name, rs[i].off);
    EXPECT(rs[i].off + rs[i].len <= p.bytes, "%s ends at %zu past %zu", rs[i].name, rs[i].off + rs[i].len, p.bytes);
    for (size_t j = 0; j < i; ++j)
      if (rs[i].len && rs[j].len)
        EXPECT(rs[i].off + rs[i].len <= rs[j].off || rs[j].off + rs[j].len <= rs[i].off, "%s overlaps %s",
               rs[i].name, rs[j].name);
  }
  // the tile table holds every tile routing can produce: sum over held
  // experts of ceil(count / bm) <= ceil(S / bm) + El (one tile per expert
  // when bm covers every expert's rows)
  const int64_t worst = d.T <= p.bm ? d.El : (S + p.bm - 1) / p.bm + d.El;
  EXPECT(p.max_tiles >= worst, "max_tiles %" PRId64 " < %" PRId64, p.max_tiles, worst);
  EXPECT(p.bm >= 8 && p.bm <= 128 && (p.bm >= 16 || p.half), "bm %" PRId64, p.bm);
  EXPECT(p.kp1 % 128 == 0 && p.kp2 % 128 == 0 && p.kp2 >= d.I && (d.I == 0 || p.kp1 >= d.H), "kp");
  const int64_t item = d.bits == 4 ? 256 : 128;
  auto split_ok = [&](const Plan::Stream& st, int64_t K, const char* name) {
    if (!st.on) return;
    EXPECT(st.splits >= 1 && st.nst >= 1, "%s splits", name);
    EXPECT((int64_t)st.splits * st.nst * st.stg * item == K, "%s: %d x %d x %d items != K %" PRId64, name,
           st.splits, st.nst, st.stg, K);
  };
  split_ok(p.s1, d.H, "FC1");
  split_ok(p.s2, d.I, "FC2");
  EXPECT(!p.small_front || (!p.share && S <= 1024 && d.E <= 1024), "small front end");
  // segment scales: tiled GEMMs whose FC2 spans (a scale block, or 128
  // codes with column scales) lie in one FC1 column tile; one segment per
  // column tile
  if (p.seg_n > 0) {
    EXPECT(p.tiled && (d.bs != 0 || d.I % 128 == 0), "segments on this shape");
    EXPECT(p.seg_shift == (d.act == QMOE_ACT_SWIGLU ? 7 : 8), "segment shift %d", p.seg_shift);
    EXPECT(p.seg_n == (d.I + (int64_t(1) << p.seg_shift) - 1) >> p.seg_shift, "segments %d", p.seg_n);
  }
  // K ranges of the tiled FC2: 1, 2 or 4, each a whole number of 256-code
  // pieces and scale blocks, at least 1024 codes; the combine sums one
  // partial set per range
  EXPECT(p.ksplit2 == 1 || p.ksplit2 == 2 || p.ksplit2 == 4, "FC2 ranges %d", p.ksplit2);
  if (p.ksplit2 > 1) {
    const int64_t kr = d.I / p.ksplit2;
    EXPECT(p.tiled && d.I % p.ksplit2 == 0 && kr % 256 == 0 && kr >= 1024 && (d.bs == 0 || kr % d.bs == 0),
           "FC2 ranges %d on I %" PRId64, p.ksplit2, d.I);
    EXPECT(p.splits2 == p.ksplit2, "partial sets %d for %d ranges", p.splits2, p.ksplit2);
  }
}

}  // namespace

// qmoe_attrs_default lives in qmoe_api.cpp with the HIP entry points; the
// defaults are restated here for the host-only build (QMoE manifest,
// attributes).
extern "C" void qmoe_attrs_default(qmoe_attrs* a) {
  std::memset(a, 0, sizeof *a);
  a->k = 1;
  a->expert_weight_bits = 4;
  a->activation_type = QMOE_ACT_RELU;
  a->activation_alpha = 1.f;
  a->routing = QMOE_ROUTE_QMOE;
  a->weights_prepacked = -1;
}

int main(int argc, char** argv) {
  const long n = argc > 1 ? std::atol(argv[1]) : 200000;
  long accepted = 0, rejected = 0;
  for (long i = 0; i < n; ++i) {
    Case c = valid_case();
    const bool mutated = next() % 3 == 0;
    if (mutated) mutate(c);
    qmoe::Dims d;
    const qmoe_status st = qmoe::validate(&c.in, &c.router, &c.w1, &c.s1, &c.w2, &c.s2,
                                          next() % 4 ? &c.out : nullptr, &c.a, &d);
    if (!mutated) EXPECT(st == QMOE_OK, "valid case %ld rejected with %d", i, (int)st);
    if (st != QMOE_OK) {
      ++rejected;
      continue;
    }
    ++accepted;
    qmoe::Plan p;
    qmoe::make_plan(d, &p);
    if (d.T > 0) check_plan(d, p);
  }
  std::printf("plan_check: %ld cases, %ld accepted, %ld rejected, %d invariant failures\n", n, accepted, rejected,
              failures);
  return failures == 0 ? 0 : 1;
}
