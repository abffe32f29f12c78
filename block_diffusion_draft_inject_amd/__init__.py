"""MI355X-native DFlash drafter block pass: C-ABI library libdflash + thin Python binding.

Importing the package loads nothing; `block_diffusion_draft_inject_amd.binding` loads the
HIP library and raises if it has not been built.
"""
