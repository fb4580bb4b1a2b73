// Host-side checks of libq8dec, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on its host code (tests/test_sanitizers.py
// builds both and runs this program on a machine without a GPU).
//
// 1. Every entry point refuses bad arguments with its named status before
//    any GPU work (the Algenta "Metal LLM decode" page's refusals with
//    status codes), and the status names cover every code.
// 2. The persistent-step planner (q8::plan_step), on the host with no
//    device (the occupancy queries fall back to one workgroup per compute
//    unit): for a set of step shapes, the workgroup groups partition the
//    tiles exactly, and the arrivals each argmax team waits for equal a
//    count taken by walking every workgroup's tiles one by one.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../include/q8dec.h"
#include "../q8_block_quantized_amd/csrc/q8dec_internal.h"

static int g_fail = 0;
#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c); \
      g_fail++;                                                         \
    }                                                                   \
  } while (0)

// aligned addresses that are never dereferenced (every call fails first)
static void *const W = (void *)0x10000;
static float *const X = (float *)0x20000;
static float *const Y = (float *)0x30000;
static int32_t *const I = (int32_t *)0x40000;

static void refusals() {
  for (int s = -3; s < 20; s++) CHECK(q8_status_name(s) != nullptr);
  CHECK(std::strcmp(q8_status_name(12), "q8_err_levels") == 0);
  CHECK(std::strcmp(q8_status_name(13), "q8_code_out_of_range") == 0);
  int32_t count = -1;
  CHECK(q8_device_count(nullptr) == Q8_ERR_NULL);
  CHECK(q8_device_count(&count) == Q8_OK && count >= 0);
  (void)q8_last_hip_error();

  CHECK(q8_matvec(nullptr, X, Y, 32, 1, nullptr) == Q8_ERR_NULL);
  CHECK(q8_matvec(W, X, Y, 33, 1, nullptr) == Q8_ERR_SHAPE);
  CHECK(q8_matvec(W, X, Y, 32, -1, nullptr) == Q8_ERR_SHAPE);
  CHECK(q8_matvec(W, X, Y, Q8_MAX_N + 32, 1, nullptr) == Q8_ERR_SHAPE);
  CHECK(q8_matvec((char *)W + 2, X, Y, 32, 1, nullptr) == Q8_ERR_ALIGN);
  CHECK(q8_matvec(W, X + 1, Y, 32, 1, nullptr) == Q8_ERR_ALIGN);
  CHECK(q8_matvec_batched(W, X, Y, 0, 32, 1, nullptr) == Q8_ERR_SHAPE);
  CHECK(q8_matvec_batched(W, X, Y, 33, 256, 1, nullptr) == Q8_ERR_SHAPE);
  CHECK(q8_matvec_batched(W, X, Y, 9, 288, 1, nullptr) == Q8_ERR_SHAPE);
  CHECK(q8_argmax(X, 0, 5, I, nullptr) == Q8_ERR_SHAPE);
  CHECK(q8_argmax(X, 1, 0, I, nullptr) == Q8_ERR_SHAPE);
  CHECK(q8_argmax(nullptr, 1, 5, I, nullptr) == Q8_ERR_NULL);
  CHECK(q8_argmax(X, 1, 5, (int32_t *)((char *)I + 2), nullptr) == Q8_ERR_ALIGN);
  CHECK(q8_matvec_argmax(W, X, nullptr, nullptr, 1, 32, 5, nullptr) == Q8_ERR_NULL);
  CHECK(q8_matvec_argmax(W, X, nullptr, I, 1, 32, 0, nullptr) == Q8_ERR_SHAPE);
  CHECK(q8_matvec_argmax_noalloc(W, X, nullptr, nullptr, 1, 32, 5, nullptr) == Q8_ERR_NULL);
  CHECK(q8_matvec_argmax_noalloc(W, X, nullptr, I, 33, 256, 5, nullptr) == Q8_ERR_SHAPE);
  CHECK(q8_matvec_i8x(W, X, Y, 1, 96, 4, nullptr) == Q8_ERR_SHAPE);
  CHECK(q8_matvec_i8x(W, X, Y, 9, 256, 4, nullptr) == Q8_ERR_SHAPE);
  CHECK(q8_matvec_argmax_i8x(W, X, nullptr, I, 1, 4096, 4, nullptr) == Q8_ERR_SHAPE);

  q8_matvec_desc d{W, X, Y, nullptr, 256, 8};
  q8_step_graph *g = (q8_step_graph *)0x1;
  CHECK(q8_step_graph_build(&d, 1, 1, nullptr, 0, nullptr, nullptr) == Q8_ERR_NULL);
  CHECK(q8_step_graph_build(nullptr, 1, 1, nullptr, 0, nullptr, &g) == Q8_ERR_NULL && !g);
  CHECK(q8_step_graph_build(&d, 0, 1, nullptr, 0, nullptr, &g) == Q8_ERR_COUNT);
  CHECK(q8_step_graph_build(&d, Q8_MAX_DESCS + 1, 1, nullptr, 0, nullptr, &g) == Q8_ERR_COUNT);
  CHECK(q8_step_graph_build(&d, 1, 1, nullptr, 7, nullptr, &g) == Q8_ERR_MODE);
  CHECK(q8_step_graph_build(&d, 1, 1, nullptr, Q8_GRAPH_LEVELS, nullptr, &g) == Q8_ERR_MODE);
  CHECK(q8_step_graph_build(&d, 1, 0, nullptr, 0, nullptr, &g) == Q8_ERR_SHAPE);
  const int32_t lv_bad[2] = {1, 0};
  q8_matvec_desc two[2] = {d, d};
  CHECK(q8_step_graph_build_levels(two, nullptr, 2, 1, nullptr, nullptr, &g) == Q8_ERR_NULL);
  CHECK(q8_step_graph_build_levels(two, lv_bad, 2, 1, nullptr, nullptr, &g) == Q8_ERR_LEVELS);
  CHECK(q8_step_graph_launch(nullptr, nullptr) == Q8_ERR_BAD_HANDLE);
  CHECK(q8_step_graph_launch_kernel(nullptr, nullptr) == Q8_ERR_BAD_HANDLE);
  CHECK(q8_step_graph_info(nullptr, nullptr, nullptr) == Q8_ERR_BAD_HANDLE);
  CHECK(q8_step_graph_destroy(nullptr) == Q8_ERR_BAD_HANDLE);
  int stack_word = 0;  // a pointer that is no handle: refused, never dereferenced
  CHECK(q8_step_graph_destroy((q8_step_graph *)&stack_word) == Q8_ERR_BAD_HANDLE);

  q8_decode_model md{};
  q8_decode_buffers bf{};
  CHECK(q8_decode_graph_build(nullptr, &bf, nullptr, nullptr, &g) == Q8_ERR_NULL);
  CHECK(q8_decode_graph_build(&md, &bf, nullptr, nullptr, nullptr) == Q8_ERR_NULL);
  CHECK(q8_decode_graph_build(&md, &bf, nullptr, nullptr, &g) == Q8_ERR_SHAPE);
  md.n_layers = 1;
  md.hidden = 1024;
  md.n_heads = 16;
  md.n_kv_heads = 8;
  md.head_dim = 64;  // only 128 is taken
  md.inter = 3072;
  md.vocab = 10;
  md.cache_rows = 64;
  md.eps = 1e-6f;
  md.theta = 1e6f;
  CHECK(q8_decode_graph_build(&md, &bf, nullptr, nullptr, &g) == Q8_ERR_SHAPE);
  md.head_dim = 128;
  md.n_heads = 40;  // 5 query heads per key/value head
  CHECK(q8_decode_graph_build(&md, &bf, nullptr, nullptr, &g) == Q8_ERR_SHAPE);
  md.n_heads = 16;
  md.eps = -1.f;
  CHECK(q8_decode_graph_build(&md, &bf, nullptr, nullptr, &g) == Q8_ERR_SHAPE);
  md.eps = 1e-6f;
  CHECK(q8_decode_graph_build(&md, &bf, nullptr, nullptr, &g) == Q8_ERR_NULL);  // no layers
}

// Walks every workgroup's tiles of a plan one by one and checks the plan.
static void check_plan(const std::vector<q8_matvec_desc> &descs, int m, int group_size,
                       bool i8x, int grid_cap = 0, uint32_t paired = 0, bool sliced = false) {
  q8::StepPlan plan;
  const int st = q8::plan_step(descs.data(), (int32_t)descs.size(), m, 0, group_size, plan, i8x,
                               grid_cap > 0 || paired, grid_cap, paired, sliced);
  CHECK(st == Q8_OK);
  if (st != Q8_OK) return;
  if (sliced) {  // 32-row tiles of 1024-wide descriptors, the sliced kernel's LDS
    CHECK(plan.lds == q8::sliced_lds_bytes(i8x) && plan.all_staged);
    for (const q8::StepDesc &t : plan.descs)
      CHECK(t.rows_per_tile == q8::sliced_rows_per_tile() && t.n == q8::kSliceWidth);
  }
  // descriptors: consecutive tile ranges covering every row
  int64_t ntiles = 0;
  for (size_t i = 0; i < descs.size(); i++) {
    const q8::StepDesc &t = plan.descs[i];
    CHECK(t.tile_begin == ntiles);
    CHECK(t.rows_per_tile >= 1);
    const int64_t tiles = ((int64_t)descs[i].p + t.rows_per_tile - 1) / t.rows_per_tile;
    CHECK(t.tile_end == t.tile_begin + tiles);
    ntiles += tiles;
  }
  CHECK(plan.grid >= 1 && plan.grid <= ntiles);
  if (grid_cap > 0) CHECK(plan.grid <= grid_cap);
  for (size_t i = 0; i < descs.size() && i < 32; i++)
    if ((paired >> i) & 1u) {
      const q8::StepDesc &t = plan.descs[i];
      CHECK(t.rows_per_tile >= 1 && t.rows_per_tile <= q8::kPairMaxRows);
      // both matrices' rows of a tile fit the staged tile buffer
      CHECK(2 * t.rows_per_tile <= q8::step_rows_per_tile(t.n, 1, false));
    }
  // groups: contiguous ranges that partition [0, ntiles); each workgroup's
  // tiles t0 + slot, + size, ... cover its group's range exactly once
  std::vector<int> owner(ntiles, -1);
  int32_t prev = 0;
  int wgs = 0;
  for (const q8::WgGroup &gr : plan.groups) {
    CHECK(gr.t0 == prev && gr.t1 >= gr.t0 && gr.first == wgs);
    CHECK(gr.size >= 1 && gr.size <= plan.group_size);
    CHECK(gr.d0 >= 0 && gr.d0 < (int32_t)descs.size());
    CHECK(plan.descs[gr.d0].tile_begin <= gr.t0);
    prev = gr.t1;
    wgs += gr.size;
    for (int j = 0; j < gr.size; j++)
      for (int64_t t = gr.t0 + q8::group_slot(j, gr.first, gr.size); t < gr.t1; t += gr.size) {
        CHECK(owner[t] == -1);
        owner[t] = gr.first + j;
      }
  }
  CHECK(prev == ntiles && wgs == plan.grid);
  for (int64_t t = 0; t < ntiles; t++) CHECK(owner[t] >= 0);
  // argmax arrivals per team: the workgroups that hold a tile of the matvec
  size_t a = 0;
  for (size_t i = 0; i < descs.size(); i++) {
    if (!descs[i].idx) continue;
    CHECK(a < plan.expected.size());
    if (a >= plan.expected.size()) return;
    std::vector<uint32_t> team(q8::kArgmaxTeams, 0);
    std::vector<char> seen(plan.grid, 0);
    for (int64_t t = plan.descs[i].tile_begin; t < plan.descs[i].tile_end; t++)
      if (!seen[owner[t]]) {
        seen[owner[t]] = 1;
        team[owner[t] % q8::kArgmaxTeams]++;
      }
    CHECK(plan.expected[a] == team);
    a++;
  }
  CHECK(a == plan.expected.size());
}

static void planner() {
  int32_t idx[8];
  auto mv = [&](int n, int p, bool argmax) {
    return q8_matvec_desc{W, X, Y, argmax ? idx : nullptr, n, p};
  };
  // the decode step's 197 matvecs, m = 1, 8 and 32
  std::vector<q8_matvec_desc> step;
  const int shapes[7][2] = {{1024, 2048}, {1024, 1024}, {1024, 1024}, {2048, 1024},
                            {1024, 3072}, {1024, 3072}, {3072, 1024}};
  for (int l = 0; l < 28; l++)
    for (auto &s : shapes) step.push_back(mv(s[0], s[1], false));
  step.push_back(mv(1024, 151936, true));
  for (int m : {1, 8, 32}) check_plan(step, m, m == 1 ? q8::kStepGroupSize : 1, false);
  check_plan(step, 1, q8::kStepGroupSize, true);
  check_plan(step, 4, 1, true);
  // ragged and empty descriptors, several argmax descriptors, odd widths
  std::vector<q8_matvec_desc> mixed = {mv(96, 0, false),  mv(256, 5, true), mv(160, 77, false),
                                       mv(1024, 1, true), mv(96, 0, false), mv(3072, 4099, true),
                                       mv(32, 3, false),  mv(2048, 17, true)};
  for (int gs : {1, 3, 8, 64}) check_plan(mixed, 1, gs, false);
  check_plan(mixed, 2, 1, false);
  // a few tiles only (the decode step's levels): heights halve to fill workgroups
  check_plan({mv(2048, 1024, false)}, 1, q8::kStepGroupSize, false);
  check_plan({mv(1024, 2048, false), mv(1024, 1024, false), mv(1024, 1024, false)}, 1,
             q8::kStepGroupSize, false);
  check_plan({mv(256, 1, true)}, 1, q8::kStepGroupSize, false);
  // the persistent decode step's phases on a grid of 512 (at most one tile
  // per workgroup where the staged heights allow), and small or odd grids
  const std::vector<std::vector<q8_matvec_desc>> phases = {
      {mv(1024, 2048, false), mv(1024, 1024, false), mv(1024, 1024, false)},
      {mv(2048, 1024, false)},
      {mv(1024, 3072, false), mv(1024, 3072, false)},
      {mv(3072, 1024, false)},
      {mv(1024, 151936, true)}};
  for (const auto &ph : phases)
    for (int cap : {512, 513, 7, 1}) check_plan(ph, 1, q8::kStepGroupSize, false, cap);
  for (int cap : {512, 3}) check_plan(mixed, 1, 8, false, cap);
  // paired gate/up descriptors (the decode step's prologue form): node form
  // and persistent grids; a paired mask with m > 1 is refused
  for (int cap : {0, 512, 7})
    check_plan({mv(1024, 3072, false)}, 1, q8::kStepGroupSize, false, cap, 1u);
  check_plan({mv(3072, 3072, false)}, 1, q8::kStepGroupSize, false, 512, 1u);
  check_plan({mv(256, 512, false), mv(1024, 77, false)}, 1, 4, false, 0, 1u);
  // the batched step in column slices: what the graph builder hands the
  // planner for the decode step at m = 8 (o and down as 2 and 3 slices;
  // binary32 and int8 activations), a ragged set with empty slices, and the
  // refusals (m = 1 either way, a slice wider than 1024)
  {
    std::vector<q8_matvec_desc> sl;
    const int slices[7][2] = {{1024, 2048}, {1024, 1024}, {1024, 1024}, {1024, 1024},
                              {1024, 3072}, {1024, 3072}, {1024, 1024}};
    const int reps[7] = {1, 1, 1, 2, 1, 1, 3};
    for (int l = 0; l < 28; l++)
      for (int k = 0; k < 7; k++)
        for (int r = 0; r < reps[k]; r++) sl.push_back(mv(slices[k][0], slices[k][1], false));
    sl.push_back(mv(1024, 151936, true));
    for (int m : {2, 8})
      for (bool i8x : {false, true}) check_plan(sl, m, 1, i8x, 0, 0u, true);
    for (bool i8x : {false, true})
      check_plan({mv(1024, 77, false), mv(1024, 0, false), mv(1024, 33, false),
                  mv(1024, 1, true)},
                 3, 1, i8x, 0, 0u, true);
    q8::StepPlan plan;
    std::vector<q8_matvec_desc> one = {mv(1024, 64, false)};
    CHECK(q8::plan_step(one.data(), 1, 1, 0, 1, plan, false, false, 0, 0u, true) == Q8_ERR_SHAPE);
    CHECK(q8::plan_step(one.data(), 1, 1, 0, 1, plan, true, false, 0, 0u, true) == Q8_ERR_SHAPE);
    std::vector<q8_matvec_desc> wide = {mv(2048, 64, false)};
    CHECK(q8::plan_step(wide.data(), 1, 8, 0, 1, plan, false, false, 0, 0u, true) == Q8_ERR_SHAPE);
  }
  {
    q8::StepPlan plan;
    std::vector<q8_matvec_desc> one = {mv(1024, 3072, false)};
    CHECK(q8::plan_step(one.data(), 1, 8, 0, 1, plan, false, true, 0, 1u) == Q8_ERR_SHAPE);
    std::vector<q8_matvec_desc> odd = {mv(96, 30, false)};
    CHECK(q8::plan_step(odd.data(), 1, 1, 0, 1, plan, false, true, 0, 1u) == Q8_ERR_SHAPE);
  }
}

int main() {
  refusals();
  planner();
  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("sanitize_driver: all checks passed\n");
  return 0;
}
