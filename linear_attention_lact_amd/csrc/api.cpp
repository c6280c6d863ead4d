// api.cpp -- status strings of the C ABI.
#include "../../include/ttt_lact.h"

extern "C" const char* ttt_status_string(ttt_status s) {
  switch (s) {
    case TTT_OK: return "ok";
    case TTT_ERR_ARG: return "invalid argument (null pointer, negative size or bad enum)";
    case TTT_ERR_SHAPE: return "inconsistent or unsupported shape";
    case TTT_ERR_UNSUPPORTED: return "combination not implemented";
    case TTT_ERR_WORKSPACE: return "workspace too small or misaligned";
    case TTT_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}
