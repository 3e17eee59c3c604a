"""Builds librs.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

    python -m linear_attention_recurrent_rs_amd.build        (or build() from Python)

Every source is compiled on each call (no caching), in parallel, then linked.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, 'csrc')
OUT = os.path.join(PKG, 'librs.so')
BUILD = os.path.join(ROOT, '_build')

HIPCC = os.environ.get('HIPCC', '/opt/rocm/bin/hipcc')
ARCH = 'gfx950'
# No packed-fp32 VALU instructions anywhere (they are disabled for all device code).
DEVICE_FLAGS = ['-Xclang', '-target-feature', '-Xclang', '-packed-fp32-ops']
COMMON = ['-O3', '-fPIC', '-std=c++17', f'--offload-arch={ARCH}', '-mcode-object-version=5',
          '-I', os.path.join(ROOT, 'include'), '-I', CSRC, '-Wall', '-Wno-unused-function']

SOURCES = ['rs_kernels.hip', 'rs_verify_fast.hip', 'rs_fold_fast.hip', 'rs_snapshot.hip',
           'rs_probe.hip', 'rs_noalloc.hip', 'rs_conv.hip', 'rs_prefill.hip', 'rs_api.cpp']


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + '.o')
    lang = ['-x', 'hip'] if src.endswith('.hip') else []
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *lang, '-c', os.path.join(CSRC, src), '-o', obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + '.tmp'
    cmd = [HIPCC, '-shared', '-fPIC', f'--offload-arch={ARCH}', *objs, '-o', tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == '__main__':
    build()
    sys.exit(0)
