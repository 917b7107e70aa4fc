// Host-only entry points of the C ABI: status strings and version.
#include "specverify.h"

extern "C" const char* spec_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_INVALID_ARG: return "invalid argument";
    case SV_ERR_UNSUPPORTED: return "unsupported shape";
    case SV_ERR_WORKSPACE: return "workspace too small";
    case SV_ERR_HIP: return "HIP runtime error";
    case SV_ERR_NO_PAGES: return "out of KV pages";
    case SV_ERR_BAD_INPUT: return "input breaks a precondition (validation mode)";
    default: return "unknown status";
  }
}

extern "C" int spec_version(void) { return 100; }
