// Host-side logic of libveda (see host.hpp). Floating-point steps mirror the
// page's Python expressions operation for operation so that budgets, splits
// and row patterns come out bit-identical to it; build with -ffp-contract=off.
#include "host.hpp"

#include "kernels.hpp"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <tuple>

namespace veda {

namespace {
thread_local std::string g_error;
}

void set_error(const std::string &msg) { g_error = msg; }
void clear_error() { g_error.clear(); }
const char *last_error() { return g_error.c_str(); }

veda_status fail(veda_status st, const std::string &msg) {
  set_error(msg);
  return st;
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t tile_count(const int32_t grid[3], const int32_t shape[3]) {
  int64_t n = 1;
  for (int i = 0; i < 3; ++i) n *= ceil_div(grid[i], shape[i]);
  return n;
}

static bool pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

bool is_box(const int32_t s[3]) {
  return pow2(s[0]) && pow2(s[1]) && pow2(s[2]) &&
         int64_t(s[0]) * s[1] * s[2] == VEDA_TILE;
}

// Minimise (tile count, max/min aspect, tuple) over the boxes that fit the
// grid on every axis, or over all 36 when none fits. The aspect is compared
// as the double max/min, as the page does.
void least_padding_shape(const int32_t grid[3], int32_t out[3]) {
  bool any_fit = false;
  for (int i = 0; i <= 7; ++i)
    for (int j = 0; i + j <= 7; ++j) {
      int32_t s[3] = {1 << i, 1 << j, 1 << (7 - i - j)};
      if (s[0] <= grid[0] && s[1] <= grid[1] && s[2] <= grid[2]) any_fit = true;
    }
  bool have = false;
  std::tuple<int64_t, double, int32_t, int32_t, int32_t> best;
  for (int i = 0; i <= 7; ++i)
    for (int j = 0; i + j <= 7; ++j) {
      int32_t s[3] = {1 << i, 1 << j, 1 << (7 - i - j)};
      bool fit = s[0] <= grid[0] && s[1] <= grid[1] && s[2] <= grid[2];
      if (any_fit && !fit) continue;
      double aspect = double(std::max({s[0], s[1], s[2]})) / double(std::min({s[0], s[1], s[2]}));
      auto key = std::make_tuple(tile_count(grid, s), aspect, s[0], s[1], s[2]);
      if (!have || key < best) {
        best = key;
        have = true;
      }
    }
  out[0] = std::get<2>(best);
  out[1] = std::get<3>(best);
  out[2] = std::get<4>(best);
}

veda_status plan_query(const veda_span *spans, int32_t n_spans, int64_t seq_len,
                       veda_plan_info *info) {
  if (!info) return fail(VEDA_ERR_INVALID, "veda_plan_query: info is NULL");
  std::memset(info, 0, sizeof(*info));
  if (n_spans <= 0 || !spans) return fail(VEDA_ERR_INVALID, "no video span given: at least one span, the generated video, is required");
  if (n_spans > VEDA_MAX_SPANS)
    return fail(VEDA_ERR_INVALID, "more than " + std::to_string(VEDA_MAX_SPANS) + " spans");
  if (seq_len <= 0 || seq_len > INT32_MAX)
    return fail(VEDA_ERR_INVALID, "seq_len must be in [1, 2^31 - 1], got " + std::to_string(seq_len));
  int64_t stop = 0, covered = 0;
  int32_t tile0 = 0;
  for (int i = 0; i < n_spans; ++i) {
    veda_span s = spans[i];
    for (int a = 0; a < 3; ++a)
      if (s.grid[a] <= 0)
        return fail(VEDA_ERR_INVALID, "span " + std::to_string(i) + ": grid sides must be positive");
    int64_t rows = int64_t(s.grid[0]) * s.grid[1] * s.grid[2];
    if (s.start < stop || s.start < 0 || s.start + rows > seq_len)
      return fail(VEDA_ERR_INVALID, "video span [" + std::to_string(s.start) + ", " +
                                        std::to_string(s.start + rows) +
                                        ") is out of packed order or outside the sequence of " +
                                        std::to_string(seq_len) + " rows");
    if (s.shape[0] == 0 && s.shape[1] == 0 && s.shape[2] == 0) {
      least_padding_shape(s.grid, s.shape);
    } else if (!is_box(s.shape)) {
      return fail(VEDA_ERR_INVALID, "span " + std::to_string(i) +
                                        ": tile box must be powers of two with t*h*w = 128");
    }
    int64_t nt = tile_count(s.grid, s.shape);
    if (int64_t(tile0) + nt > INT32_MAX / VEDA_TILE)
      return fail(VEDA_ERR_INVALID, "too many tiles");
    info->spans[i] = s;
    info->span_tile0[i] = tile0;
    tile0 += int32_t(nt);
    stop = s.start + rows;
    covered += rows;
    if (i + 1 < n_spans) info->ref_tokens += rows;
    else info->target_tokens = rows;
  }
  info->span_tile0[n_spans] = tile0;
  info->n_spans = n_spans;
  info->seq_len = seq_len;
  info->n_video = tile0;
  info->n_ref = info->span_tile0[n_spans - 1];
  info->global_rows = seq_len - covered;
  info->n_global = int32_t(ceil_div(info->global_rows, VEDA_TILE));
  info->n_tiles = info->n_video + info->n_global;
  info->n_slots = int64_t(info->n_tiles) * VEDA_TILE;
  clear_error();
  return VEDA_OK;
}

// Python: budget[0] * ideal * ideal / n_cols, ideal = math.ceil(real / 128).
// real / 128 is exact in doubles, so ceil of it is the integer ceiling.
double per_row(veda_budget b, int64_t real_tokens, int32_t n_cols) {
  if (b.tiles >= 0.0) return b.tiles;
  double ideal = double(ceil_div(real_tokens, VEDA_TILE));
  double x = b.ratio * ideal;
  x = x * ideal;
  return x / double(n_cols);
}

// Python's round(x, 12): the double nearest the decimal that is x correctly
// rounded to 12 places. printf's %.12f rounds the exact binary value
// correctly and strtod reads a decimal back correctly, which is the same pair
// of steps.
double round12(double x) {
  char buf[64];
  std::snprintf(buf, sizeof(buf), "%.12f", x);
  return std::strtod(buf, nullptr);
}

void split(double b, int32_t n, int32_t *lo, int32_t *hi, double *frac) {
  if (b >= double(n)) {
    *lo = n;
    *hi = n;
    *frac = 0.0;
    return;
  }
  double fl = std::floor(b);
  int64_t l = std::min<int64_t>(std::max<int64_t>(1, int64_t(fl)), n);
  *lo = int32_t(l);
  *hi = int32_t(std::min<int64_t>(l + 1, n));
  double f = b - double(l);
  f = std::min(std::max(f, 0.0), 1.0);
  *frac = round12(f);
}

bool bresenham_extra(int64_t r, double frac) {
  double a = std::floor(double(r + 1) * frac);
  double b = std::floor(double(r) * frac);
  return a > b;
}

int64_t row_offset(const veda_plan_info *info, const veda_select_info *sel, int64_t r) {
  int64_t nv = info->n_video;
  int64_t rv = std::min<int64_t>(r, nv);
  int64_t off = 0;
  for (int b = 0; b < sel->n_blocks; ++b) {
    const veda_block &k = sel->blocks[b];
    if (k.keep_all) off += rv * int64_t(k.stop - k.start);
    else off += rv * int64_t(k.k_lo) + int64_t(std::floor(double(rv) * k.frac));
  }
  off += rv * int64_t(info->n_global);
  if (r > nv) off += (r - nv) * int64_t(info->n_tiles);
  return off;
}

static veda_status check_budget(veda_budget b, const char *what) {
  bool r = b.ratio >= 0.0, t = b.tiles >= 0.0;
  if (r == t)
    return fail(VEDA_ERR_INVALID, std::string(what) + " budget: set exactly one of ratio, tiles");
  if (!std::isfinite(r ? b.ratio : b.tiles))
    return fail(VEDA_ERR_INVALID, std::string(what) + " budget must be finite");
  return VEDA_OK;
}

veda_status select_query(const veda_plan_info *info, veda_budget generated,
                         veda_budget reference, int32_t head_dim, int32_t n_heads,
                         veda_select_info *sel) {
  if (!info || !sel) return fail(VEDA_ERR_INVALID, "veda_select_query: NULL argument");
  std::memset(sel, 0, sizeof(*sel));
  if (info->n_spans <= 0 || info->n_video <= 0)
    return fail(VEDA_ERR_INVALID, "plan info is empty (call veda_plan_query first)");
  if (head_dim != 64 && head_dim != 128)
    return fail(VEDA_ERR_UNSUPPORTED, "head_dim must be 64 or 128, got " + std::to_string(head_dim));
  if (n_heads <= 0 || n_heads > VEDA_MAX_HEADS)
    return fail(VEDA_ERR_INVALID, "n_heads must be in [1, " + std::to_string(VEDA_MAX_HEADS) + "]");
  veda_status st = check_budget(generated, "generated");
  if (st != VEDA_OK) return st;
  // Column blocks: the reference tiles (when there are any) and the target
  // each take their own top-k (section "selection", column_blocks).
  struct Req { int32_t start, stop; veda_budget b; int64_t real; };
  Req reqs[VEDA_MAX_BLOCKS];
  int nb = 0;
  if (info->n_ref > 0) {
    st = check_budget(reference, "reference");
    if (st != VEDA_OK) return st;
    reqs[nb++] = {0, info->n_ref, reference, info->ref_tokens};
  }
  reqs[nb++] = {info->n_ref, info->n_video, generated, info->target_tokens};
  sel->n_blocks = nb;
  sel->head_dim = head_dim;
  sel->n_heads = n_heads;
  int64_t widest_video = info->n_global;
  for (int b = 0; b < nb; ++b) {
    veda_block &k = sel->blocks[b];
    const Req &q = reqs[b];
    int32_t n = q.stop - q.start;
    k.start = q.start;
    k.stop = q.stop;
    // keeps_all: a ratio budget of at least 1 (a tile budget never is).
    k.keep_all = (q.b.tiles < 0.0 && q.b.ratio >= 1.0) ? 1 : 0;
    if (k.keep_all) {
      k.k_lo = k.k_hi = n;
      k.frac = 0.0;
      widest_video += n;
      continue;
    }
    split(per_row(q.b, q.real, n), n, &k.k_lo, &k.k_hi, &k.frac);
    // The CSR row starts use sum_{r'<r} extra(r') = floor(r * frac), which
    // holds when floor(r * frac) never steps by more than one.
    double prev = 0.0;
    for (int64_t r = 1; r <= info->n_video; ++r) {
      double cur = std::floor(double(r) * k.frac);
      if (cur - prev > 1.0)
        return fail(VEDA_ERR_UNSUPPORTED, "budget fraction too close to 1 for the row pattern");
      prev = cur;
    }
    widest_video += (k.frac > 0.0 ? std::min(k.k_lo + 1, n) : k.k_lo);
  }
  sel->widest = int32_t(info->n_global > 0 ? std::max<int64_t>(widest_video, info->n_tiles)
                                           : widest_video);
  sel->entries_per_head = row_offset(info, sel, info->n_tiles);
  if (int64_t(n_heads) * sel->entries_per_head > INT32_MAX)
    return fail(VEDA_ERR_UNSUPPORTED, "tile lists of all heads exceed 2^31 entries");
  sel->workspace_bytes = select_workspace(info, head_dim, n_heads).total;
  clear_error();
  return VEDA_OK;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

SelectWorkspace select_workspace(const veda_plan_info *info, int32_t D, int32_t H) {
  SelectWorkspace w;
  size_t nv = size_t(info->n_video);
  w.feat_off = 0;
  w.feat_bytes = align256(2 * size_t(H) * nv * 3 * D * sizeof(double));
  w.proj_off = w.feat_off + w.feat_bytes;
  w.proj_bytes = align256(2 * size_t(H) * nv * D * sizeof(double));
  w.score_off = w.proj_off + w.proj_bytes;
  w.score_bytes = align256(size_t(H) * nv * nv * sizeof(double));
  w.total = w.score_off + w.score_bytes;
  return w;
}

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

veda_status check_info(const veda_plan_info *info) {
  if (!info || info->n_spans <= 0 || info->n_spans > VEDA_MAX_SPANS || info->n_video <= 0 ||
      info->n_tiles < info->n_video)
    return fail(VEDA_ERR_INVALID, "plan info is empty or corrupt (call veda_plan_query)");
  return VEDA_OK;
}

// Tensors the kernels read 16 bytes at a time: base and both strides must keep
// every row 16-byte aligned.
veda_status check_tensor(const void *p, veda_dtype dt, int64_t ss, int64_t sh, const char *name) {
  if (!p) return fail(VEDA_ERR_INVALID, std::string(name) + " is NULL");
  const int64_t elt = dt == VEDA_BF16 ? 2 : 4;
  if (!aligned16(p) || (ss * elt) % 16 != 0 || (sh * elt) % 16 != 0)
    return fail(VEDA_ERR_UNSUPPORTED,
                std::string(name) + ": base and strides must be 16-byte aligned");
  return VEDA_OK;
}

veda_status fill_heads(const int32_t *heads, int32_t n_heads, int32_t n_heads_total,
                       HeadList *hl) {
  if (!heads) return fail(VEDA_ERR_INVALID, "heads is NULL");
  if (n_heads <= 0 || n_heads > VEDA_MAX_HEADS)
    return fail(VEDA_ERR_INVALID, "n_heads out of range");
  std::memset(hl, 0, sizeof(*hl));
  for (int i = 0; i < n_heads; ++i) {
    if (heads[i] < 0 || heads[i] >= n_heads_total)
      return fail(VEDA_ERR_INVALID, "head index " + std::to_string(heads[i]) + " not in [0, " +
                                        std::to_string(n_heads_total) + ")");
    hl->h[i] = heads[i];
  }
  return VEDA_OK;
}

veda_status attend_prepare(const veda_plan_info *info, const veda_select_info *sel,
                           const int32_t *perm, const int32_t *valid_count, const void *q,
                           const void *k, const void *v, void *out, veda_dtype dtype,
                           int64_t stride_s, int64_t stride_h, int64_t out_stride_s,
                           int64_t out_stride_h, int32_t n_heads_total, const int32_t *heads,
                           const int32_t *row_offsets, const int32_t *cols, float scale,
                           AttendArgs *a, HeadList *hl) {
  veda_status st = check_info(info);
  if (st != VEDA_OK) return st;
  if (!sel || sel->n_blocks <= 0)
    return fail(VEDA_ERR_INVALID, "select info is empty (call veda_select_query)");
  if (!perm || !valid_count || !row_offsets || !cols)
    return fail(VEDA_ERR_INVALID, "perm / valid_count / row_offsets / cols is NULL");
  if (dtype != VEDA_F32 && dtype != VEDA_BF16) return fail(VEDA_ERR_INVALID, "unknown dtype");
  const int D = sel->head_dim;
  if (D != 64 && D != 128) return fail(VEDA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if ((st = check_tensor(q, dtype, stride_s, stride_h, "q")) != VEDA_OK) return st;
  if ((st = check_tensor(k, dtype, stride_s, stride_h, "k")) != VEDA_OK) return st;
  if ((st = check_tensor(v, dtype, stride_s, stride_h, "v")) != VEDA_OK) return st;
  if ((st = check_tensor(out, dtype, out_stride_s, out_stride_h, "out")) != VEDA_OK) return st;
  st = fill_heads(heads, sel->n_heads, n_heads_total, hl);
  if (st != VEDA_OK) return st;
  // K/V rows are read with 32-bit offsets from each head's first element.
  const int64_t elt = dtype == VEDA_BF16 ? 2 : 4;
  const int64_t kv_extent = ((info->seq_len - 1) * stride_s + D) * elt;
  if (dtype == VEDA_BF16 && kv_extent > int64_t(0xE0000000))
    return fail(VEDA_ERR_UNSUPPORTED, "q/k/v rows of one head span more than 3.5 GiB");
  // Row offsets are formed as row * pitch + chunk with 24-bit factors; a
  // padding slot is read as row seq_len, which must fall past the range above
  // (rows may not overlap) and still fit in 32 bits.
  if (dtype == VEDA_BF16 && (stride_s < D || stride_s * 2 >= (int64_t(1) << 24) ||
                             info->seq_len >= (int64_t(1) << 24) ||
                             (info->seq_len + 1) * stride_s * 2 > int64_t(0xFFFFFFFF)))
    return fail(VEDA_ERR_UNSUPPORTED,
                "bf16 attend needs D <= stride_s < 2^23 elements and seq_len < 2^24 rows");
  if (!(scale > 0.0f)) scale = float(1.0 / std::sqrt(double(D)));
  std::memset(a, 0, sizeof(*a));
  a->q = q;
  a->k = k;
  a->v = v;
  a->out = out;
  a->stride_s = stride_s;
  a->stride_h = stride_h;
  a->out_stride_s = out_stride_s;
  a->out_stride_h = out_stride_h;
  a->perm = perm;
  a->valid_count = valid_count;
  a->row_offsets = row_offsets;
  a->cols = cols;
  a->entries_per_head = sel->entries_per_head;
  a->n_heads = sel->n_heads;
  a->n_tiles = info->n_tiles;
  a->n_video = info->n_video;
  a->kv_bytes = uint32_t(kv_extent);
  a->pad_row = uint32_t(info->seq_len);
  a->scale = scale;
  a->scale_log2 = float(double(scale) * 1.4426950408889634);
  return VEDA_OK;
}

veda_status int8_workspace(const veda_plan_info *info, const veda_select_info *sel,
                           Int8Workspace *w) {
  veda_status st = check_info(info);
  if (st != VEDA_OK) return st;
  if (!sel || sel->n_blocks <= 0)
    return fail(VEDA_ERR_INVALID, "select info is empty (call veda_select_query)");
  if (sel->head_dim != 64 && sel->head_dim != 128)
    return fail(VEDA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  const int64_t per_head = int64_t(info->n_tiles) * VEDA_TILE * sel->head_dim;
  if (per_head >= (int64_t(1) << 31))
    return fail(VEDA_ERR_UNSUPPORTED, "one head's int8 K codes reach 2 GiB");
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  w->codes_off = 0;
  w->codes_bytes = size_t(per_head) * size_t(sel->n_heads);
  w->scale_off = up(w->codes_bytes);
  w->scale_bytes = sizeof(float) * size_t(info->n_tiles) * size_t(sel->n_heads);
  w->total = up(w->scale_off + w->scale_bytes);
  return VEDA_OK;
}

}  // namespace veda
