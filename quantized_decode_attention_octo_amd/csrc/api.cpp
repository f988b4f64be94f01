// C-ABI plumbing of the OCTOPUS library: version, status strings, the
// thread-local error message and the host-side validation shared by the
// entry points.  Nothing here touches the device.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cmath>
#include <cstring>

#include "octo_internal.h"

namespace octo {

static thread_local char g_msg[512];

octo_status fail(octo_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof g_msg, fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_msg[0] = 0; }

// The splits every kernel is compiled for: the paper's (b+1, b-1) default for
// b = 2, 3, 4 (Sec. 3.3, 3.4: at most 32 + 8 centroids) and the uniform (b, b)
// reference for the same b.
static bool split_supported(int bd, int bn) {
  static const int ok[][2] = {{3, 1}, {4, 2}, {5, 3}, {2, 2}, {3, 3}, {4, 4}};
  for (auto& p : ok)
    if (p[0] == bd && p[1] == bn) return true;
  return false;
}

// The rest of the (b + delta, b - delta) sweep of Sec. 3.3 (Empirical
// verification: b = 2, 3, 4, delta = -2 .. 2), for the encoder and the
// explicit reconstruction only.
static bool sweep_split(int bd, int bn) {
  const int b = (bd + bn) / 2, delta = bd - b;
  return (bd + bn) % 2 == 0 && b >= 2 && b <= 4 && delta >= -2 && delta <= 2;
}

octo_status resolve_codec(const octo_codec_desc* d, const char* what, Codec* out,
                          bool need_tables, bool any_split) {
  if (!d) return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: codec descriptor is NULL", what);
  if (d->abi_version != OCTO_ABI_VERSION)
    return fail(OCTO_ERR_VERSION, "%s: descriptor abi_version %u, library %u", what,
                d->abi_version, OCTO_ABI_VERSION);
  if (d->head_dim <= 0 || (d->head_dim & (d->head_dim - 1)))
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: head_dim %d is not a power of two", what,
                d->head_dim);
  if (d->head_dim != kHeadDim)
    return fail(OCTO_ERR_UNSUPPORTED, "%s: head_dim %d (only 128 is compiled)", what, d->head_dim);
  if (d->group != 0) {
    // the group-wise value codec: codes, E4M3 scales and BF16 zero-points
    if (d->group < 0) return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: group %d is negative", what, d->group);
    if (d->group != 16 && d->group != 32)
      return fail(OCTO_ERR_UNSUPPORTED, "%s: group size %d (16 and 32 are compiled)", what, d->group);
    if (d->bits < 1 || d->bits > 8)
      return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: bits %d out of range", what, d->bits);
    if (d->bits < 2 || d->bits > 4)
      return fail(OCTO_ERR_UNSUPPORTED, "%s: group codec bits %d (2, 3 and 4 are compiled)", what,
                  d->bits);
    if (d->b_dir != 0 || d->b_nrm != 0)
      return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: b_dir and b_nrm must be 0 with a group codec", what);
    if (d->qjl != 0)
      return fail(OCTO_ERR_UNSUPPORTED, "%s: the group codec carries no QJL sketch", what);
    Codec g;
    std::memset(&g, 0, sizeof(g));
    g.group = d->group;
    g.bits = d->bits;
    g.w_idx = group_record_words(d->bits, d->group);
    g.seed = d->seed;
    *out = g;
    return OCTO_OK;
  }
  int bd = d->b_dir, bn = d->b_nrm;
  if (bd == 0 && bn == 0) {
    if (d->bits < 1 || d->bits > 8)
      return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: bits %d out of range", what, d->bits);
    bd = d->bits + 1;
    bn = d->bits - 1;
  }
  if (bd < 0 || bn < 0 || bd > 8 || bn > 8)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: split (%d, %d) out of range", what, bd, bn);
  if (!split_supported(bd, bn) && !(any_split && sweep_split(bd, bn)))
    return fail(OCTO_ERR_UNSUPPORTED, "%s: split (b_dir %d, b_nrm %d) not compiled", what, bd, bn);
  if (d->rounding != OCTO_ROUND_LOCAL3X3 && d->rounding != OCTO_ROUND_SCALAR)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: rounding %d unknown", what, d->rounding);
  if (d->qjl != 0 && d->qjl != 1)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: qjl must be 0 or 1", what);
  Codebook cb;
  WideCodebook wcb;
  std::memset(&cb, 0, sizeof(cb));
  std::memset(&wcb, 0, sizeof(wcb));
  if (need_tables) {
    if (!d->c_xi || !d->c_rho)
      return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: codebook pointer is NULL", what);
    if (((uintptr_t)d->c_xi | (uintptr_t)d->c_rho) & 3)
      return fail(OCTO_ERR_ALIGNMENT, "%s: codebooks must be 4-byte aligned", what);
    std::memcpy(wcb.xi, d->c_xi, sizeof(float) << bd);
    std::memcpy(wcb.rho, d->c_rho, sizeof(float) << bn);
    for (int i = 0; i < (1 << bd); ++i)
      if (!std::isfinite(wcb.xi[i]) || (i > 0 && !(wcb.xi[i] > wcb.xi[i - 1])))
        return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: c_xi is not finite and ascending", what);
    for (int i = 0; i < (1 << bn); ++i)
      if (!std::isfinite(wcb.rho[i]) || (i > 0 && !(wcb.rho[i] > wcb.rho[i - 1])))
        return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: c_rho is not finite and ascending", what);
    if (bd <= 5 && bn <= 4) {
      std::memcpy(cb.xi, wcb.xi, sizeof(float) << bd);
      std::memcpy(cb.rho, wcb.rho, sizeof(float) << bn);
    }
  }
  out->group = 0;
  out->bits = (bd + bn) / 2;
  out->b_dir = bd;
  out->b_nrm = bn;
  out->K = 1 << bd;
  out->R = 1 << bn;
  out->w_idx = words_for_bits(kNTri * (2 * bd + bn));
  out->w_qjl = d->qjl ? words_for_bits(kHeadDim) : 0;
  out->qjl = d->qjl;
  out->rounding = d->rounding;
  out->seed = d->seed;
  out->cb = cb;
  out->wcb = wcb;
  return OCTO_OK;
}

octo_status check_cache(const octo_cache_view* v, const Codec& c, const char* what) {
  if (!v) return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: cache view is NULL", what);
  if (v->layout != OCTO_LAYOUT_TILE64)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: layout %d unknown", what, v->layout);
  if (v->batch < 1 || v->kv_heads < 1 || v->capacity < 0)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: batch %d, kv_heads %d, capacity %d", what,
                v->batch, v->kv_heads, v->capacity);
  if (v->capacity % 64)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: capacity %d is not a multiple of 64", what,
                v->capacity);
  if (!v->idx || (!c.group && !v->gamma))
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: stream pointer is NULL", what);
  if (c.qjl && (!v->qjl || !v->gamma_r))
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: QJL codec needs qjl and gamma_r streams", what);
  uintptr_t a = (uintptr_t)v->idx | (c.group ? 0 : (uintptr_t)v->gamma);
  if (c.qjl) a |= (uintptr_t)v->qjl;
  if (a & 15) return fail(OCTO_ERR_ALIGNMENT, "%s: streams must be 16-byte aligned", what);
  if (c.qjl && ((uintptr_t)v->gamma_r & 1))
    return fail(OCTO_ERR_ALIGNMENT, "%s: gamma_r must be 2-byte aligned", what);
  return OCTO_OK;
}

octo_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(OCTO_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return OCTO_OK;
}

}  // namespace octo

extern "C" {

uint32_t octo_abi_version(void) { return OCTO_ABI_VERSION; }

const char* octo_status_string(int32_t s) {
  switch (s) {
    case OCTO_OK: return "OCTO_OK";
    case OCTO_ERR_INVALID_ARGUMENT: return "OCTO_ERR_INVALID_ARGUMENT";
    case OCTO_ERR_UNSUPPORTED: return "OCTO_ERR_UNSUPPORTED";
    case OCTO_ERR_ALIGNMENT: return "OCTO_ERR_ALIGNMENT";
    case OCTO_ERR_CAPACITY: return "OCTO_ERR_CAPACITY";
    case OCTO_ERR_WORKSPACE_TOO_SMALL: return "OCTO_ERR_WORKSPACE_TOO_SMALL";
    case OCTO_ERR_VERSION: return "OCTO_ERR_VERSION";
    case OCTO_ERR_HIP: return "OCTO_ERR_HIP";
  }
  return "OCTO_ERR_UNKNOWN";
}

const char* octo_last_error(void) { return octo::g_msg; }

octo_status octo_record_sizes(const octo_codec_desc* codec, octo_stream_sizes* out) {
  octo::clear_error();
  if (!out) return octo::fail(OCTO_ERR_INVALID_ARGUMENT, "octo_record_sizes: out is NULL");
  octo::Codec c;
  octo_status s = octo::resolve_codec(codec, "octo_record_sizes", &c, false, true);
  if (s != OCTO_OK) return s;
  out->idx_words = c.w_idx;
  out->qjl_words = c.w_qjl;
  out->n_triplets = c.group ? 0 : octo::kNTri;
  out->b_dir = c.b_dir;
  out->b_nrm = c.b_nrm;
  return OCTO_OK;
}

}  // extern "C"
