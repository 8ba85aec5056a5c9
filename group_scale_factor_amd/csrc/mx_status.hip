// Status texts of the C ABI (host code only; no kernels here, so that host-side
// edits leave the kernel sources untouched).

#include <stdint.h>

#include "mx_rearrange.h"

extern "C" {

const char *mx_rearrange_strerror(int status) {
  switch (status) {
    case MX_REARRANGE_OK: return "success";
    case MX_REARRANGE_ENULL: return "a required pointer is NULL";
    case MX_REARRANGE_ESHAPE: return "invalid shape or stride: negative, too large, or a row stride out of its range";
    case MX_REARRANGE_EGROUPS: return "num_groups out of range (at least 1; the casts also cap it)";
    case MX_REARRANGE_EALIGN: return "a buffer or row stride is not aligned as the entry point requires";
    case MX_REARRANGE_ELAUNCH: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
